// Frame-wise Gated DeltaNet forward, bf16 I/O: the Gram form on gfx950.
//
// The write of one frame (SANA-WM news article "NVIDIA Apresenta SANA-WM ...",
// section "1. Atencao Linear Hibrida com Gated DeltaNet (GDN)") expands, with
// Kf = ReLU(K_t)/sqrt(D*S), to
//   M_t = g M + Kf^T V - b g (Kf^T Kf) M          (ERASE)
//   M_t = g M + b Kf^T V - b g (Kf^T Kf) M        (WRITE)
// so everything that touches the S tokens of a frame -- the D x D Gram matrix
// G_t = Kf^T Kf and the D x D input term B_t = Kf^T V -- depends on that frame
// alone.  The forward then runs in three passes:
//   gdn_gram   (all frames in parallel, HBM-bound): G_t and B_t per (head,
//              frame) from one read of K_t and V_t, stored as bf16 in the
//              exact register layouts the next pass consumes;
//   gdn_state  (serial over frames, tiny): M_t = g M - b g G_t bf16(M) + B_t
//              (B_t scaled by b in WRITE mode), one D x D product per frame,
//              plus the bf16 snapshot of M_t;
//   gdn_readout (all frames in parallel, HBM-bound; gdn_kernels.hip):
//              O_t = ReLU(Q_t) M_t from the snapshots, and the state norms
//              from the same bf16 snapshots.
// Only the second pass is sequential, and it reads 2*D*D*2 bytes per frame
// instead of the frame's 2*S*D*2 bytes of keys and values.
//
// Layouts (see gdn_device.h for the MFMA lane maps).  The Gram pass builds
// its operands with transposed LDS reads, so the 8 k-slots of lane (i, g) of a
// 32-token chunk hold tokens 4g..4g+3 and 16+4g..16+4g+3.  Its accumulator
// C(L, I) for 16-key blocks L and I therefore holds, in lane (b, g),
// G[16L + 4g + r][16I + b] for r = 0..3.  G is symmetric, so only the blocks
// (I, L) with I >= L are stored, each as a 16 x 16 bf16 tile of 512 bytes in
// which the 4 elements (row x, columns 4c..4c+3) sit at byte (16c + x) * 8:
// by symmetry block (I, L) is C(L, I) read with rows and columns swapped, so
// lane l = 16g + b of C(L, I) owns exactly bytes 8l..8l+7 of block (I, L) --
// one store of 512 contiguous bytes in lane order.  The state pass uses the
// k-slot order over
// keys in which slot e of lane group g in k-step kb is key
// 32kb + 16(e/4) + 4g + e%4.  Its A operand for output block I and k-step kb
// takes, in lane (a, g), row a, columns 4g..4g+3 of the blocks (I, 2kb) and
// (I, 2kb+1): a plain 8-byte read from a stored block when I >= L, and a
// transposed 8-byte LDS read (ds_read_b64_tr_b16) from the stored block
// (L, I) when L > I.  In the same order the state pass's B operand is its own
// accumulator layout (lane (n, g) holds M[16I + 4g + r][n]), so the bf16 copy
// of the state exchanged each frame is lane-linear, 8 bytes per lane per block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// ----------------------------------------------------------------------------
// Gram pass.  One workgroup per (head, frame).  Its output is the NB*NB blocks
// of B = Kf^T V and the NB(NB+1)/2 stored blocks (I >= L) of G = Kf^T Kf, in
// 16 x 16 blocks (NB = D/16); the list of output blocks is cut into equal
// contiguous ranges, one per wave, fixed at compile time.  The frame's tokens
// are walked in 32-token chunks: each chunk of K and V is loaded once
// (coalesced 1 KB loads spread over the waves, kept kGramRing chunks ahead in
// registers), passed through ReLU (keys) and staged in a double-buffered LDS
// tile, from which every wave takes the operands its blocks need with
// transposed reads, one MFMA per block and chunk.  With e4m3 I/O the tile
// holds the codes themselves (keys through a sign-bit ReLU) and the blocks
// are 16x16x32 fp8 MFMAs: the products are those of the decoded values, the
// 32-term sum inside the instruction is not rounded once to fp32 (on gfx950
// it lands within about 2^-12 of the sum of |products| of the exact value).
// ----------------------------------------------------------------------------
constexpr int kGramRing = 4;   // chunks in flight per workgroup (even: LDS buffer = slot % 2)

template <int D>
struct GramShape {
  static constexpr int NB = D / 16;                   // 16-key (and 16-value) blocks
  static constexpr int NKC = (NB + 1) / 2;            // 32-key k-steps of the state product
  static constexpr int NW = (NB + 1) / 2;             // waves
  static constexpr int UPR = D / 8;                   // 16-byte units per token row
  static constexpr int NLD = D / 16;                  // 1 KB pieces per 32-token chunk of one tensor
  static constexpr int LPW = (2 * NLD + NW - 1) / NW; // pieces loaded per wave per chunk
  static constexpr int RS = D + 8;                    // LDS row stride (elements)
  static constexpr int RS8 = D + 8;                   // row stride of an e4m3 tile (bytes)
  static constexpr size_t tile_bytes = (size_t)32 * RS * 2;
  static constexpr size_t lds_bytes = 2 * 2 * tile_bytes;   // (K, V) x 2 buffers
  static constexpr int NBLK = NB * (NB + 1) / 2;       // stored G blocks (I >= L)
  static constexpr int NBB = NB * NB;                  // B blocks
  static constexpr int NOUT = NBB + NBLK;              // output blocks: B blocks, then G blocks
  static constexpr size_t g_frame_bytes = (size_t)(NBLK + 1) / 2 * 1024;   // per (head, frame), 1 KB units
  static constexpr size_t b_frame_bytes = (size_t)NB * NB * 512;
};

// stored G block k = I(I+1)/2 + L (I >= L) -> I, L
constexpr int gblk_row(int k) {
  int I = 0;
  while ((I + 1) * (I + 2) / 2 <= k) ++I;
  return I;
}
constexpr int gblk_col(int k) { return k - gblk_row(k) * (gblk_row(k) + 1) / 2; }

// Output block b of the gram pass: b < NBB is B block (value block j = b / NB,
// key block L = b % NB), accumulated as MFMA(X_L, Y_j); b >= NBB is stored G
// block k = b - NBB = (I, L), accumulated as MFMA(X_L, X_I) = C(L, I).
// Bit masks of the key (X) and value (Y) operand blocks that the output
// blocks [b0, b1) use.
constexpr uint32_t gram_xmask(int NB, int b0, int b1) {
  uint32_t m = 0;
  for (int b = b0; b < b1; ++b) {
    if (b < NB * NB) {
      m |= 1u << (b % NB);
    } else {
      m |= 1u << gblk_row(b - NB * NB);
      m |= 1u << gblk_col(b - NB * NB);
    }
  }
  return m;
}
constexpr uint32_t gram_ymask(int NB, int b0, int b1) {
  uint32_t m = 0;
  for (int b = b0; b < b1 && b < NB * NB; ++b) m |= 1u << (b / NB);
  return m;
}

// NW waves share a frame's output blocks and its loads (GramShape<D>::NW, or
// twice that for launches too small to fill the GPU, where the time of one
// workgroup is the latency of the whole launch).  Every block is accumulated
// over the chunks in the same order whatever NW is, so the bits do not change.
template <int D, bool FP8, int NW, int W, int CPI>
__device__ __forceinline__ void gram_wave(const GramArgs& a, unsigned char* smem, int bh, int tl) {
  using Sh = GramShape<D>;
  using IO = IoFmt<FP8>;
  constexpr int NB = Sh::NB, UPR = Sh::UPR, NLD = Sh::NLD, RS = Sh::RS;
  constexpr int LPW = (2 * NLD + NW - 1) / NW;        // pieces loaded per wave per chunk
  constexpr int NBB = Sh::NBB, NOUT = Sh::NOUT;
  constexpr int B0 = W * NOUT / NW, B1 = (W + 1) * NOUT / NW, NMB = B1 - B0;   // my output blocks
  constexpr uint32_t XM = gram_xmask(NB, B0, B1), YM = gram_ymask(NB, B0, B1);
  const int l = lane_id(), g = l >> 4, n = l & 15;
  const int S = a.S, T = a.T, t = a.t0 + tl;
  const uint32_t head_bytes = (uint32_t)T * (uint32_t)S * D * IO::ebytes;
  const size_t head0 = (size_t)bh * T * S * D * IO::ebytes;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc((const unsigned char*)a.k + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const unsigned char*)a.v + head0, head_bytes);
  const uint32_t fbyte = (uint32_t)t * (uint32_t)S * D * IO::ebytes;
  const int nch = (S + 31) / 32;
  const int nit = (nch + kGramRing - 1) / kGramRing * kGramRing;
  using raw = typename IO::raw;

  // piece p of a chunk: p < NLD are keys, NLD <= p < 2 NLD values; lane l of
  // piece p carries 8-element unit 64 (p mod NLD) + l of the chunk.
  auto load_chunk = [&](int ch, raw (&X)[LPW]) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int p = W + NW * i;
      const int u = 64 * (p % NLD) + l;
      const int tok = ch * 32 + u / UPR;
      const bool ok = p < 2 * NLD && ch < nch && tok < S;
      const uint32_t off = ok ? fbyte + (uint32_t)(ch * 32 * UPR + u) * IO::unit_bytes : kOOB;
      X[i] = IO::load_nt(p < NLD ? krs : vrs, off);
    }
  };
  // bf16 I/O: staged as bf16 (K through ReLU), bf16 MFMAs; e4m3 I/O:
  // staged as e4m3 codes, e4m3 MFMAs on the exact codes
  auto stage = [&](int buf, const raw (&X)[LPW]) {
    if constexpr (FP8) {
      unsigned char* kt = smem + (size_t)buf * 2 * Sh::tile_bytes;
      unsigned char* vt = kt + 32 * Sh::RS8;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int p = W + NW * i;
        if (p < 2 * NLD) {
          const int u = 64 * (p % NLD) + l;
          unsigned char* dst = (p < NLD ? kt : vt) + (u / UPR) * Sh::RS8 + 8 * (u % UPR);
          *(u32x2*)dst = p < NLD ? relu_e4m3x8(X[i]) : X[i];
        }
      }
    } else {
      uint16_t* kt = (uint16_t*)(smem + (size_t)buf * 2 * Sh::tile_bytes);
      uint16_t* vt = kt + 32 * RS;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int p = W + NW * i;
        if (p < 2 * NLD) {
          const int u = 64 * (p % NLD) + l;
          uint16_t* dst = (p < NLD ? kt : vt) + (u / UPR) * RS + 8 * (u % UPR);
          const u32x4 x = IO::to_bf16(X[i]);
          *(u32x4*)dst = p < NLD ? relu8(x) : x;
        }
      }
    }
  };
  // operand of 16-column block `blk` of a staged tile: lane (i, g) gets column
  // 16 blk + i at tokens 4g..4g+3 and 16+4g..16+4g+3
  auto frag = [&](const uint16_t* tile, int blk) -> u32x4 {
    const uint16_t* p0 = tile + (4 * g + (n >> 2)) * RS + 16 * blk + 4 * (n & 3);
    const u32x2 x = lds_tr16(p0), y = lds_tr16(p0 + 16 * RS);
    return u32x4{x[0], x[1], y[0], y[1]};
  };
  // e4m3 operand of block blk: lane l gets dim 16 blk + l % 16 of tokens
  // 8 (l / 16) .. + 7, the 16 lanes of a group naming rows (token, 8-byte
  // half) for the transposing read
  auto frag8 = [&](const unsigned char* tile, int blk) -> u32x2 {
    return lds_tr8(tile + (8 * g + (n >> 1)) * Sh::RS8 + 16 * blk + 8 * (n & 1));
  };

  f32x4 acc[NMB];
#pragma unroll
  for (int i = 0; i < NMB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  raw R[kGramRing][LPW];
#pragma unroll
  for (int r = 0; r < kGramRing; ++r) load_chunk(r, R[r]);

  // CPI chunks are staged per barrier, into buffer set (slot / CPI) % 2
  static_assert(kGramRing % (2 * CPI) == 0, "the LDS buffer sets alternate within the ring");
  for (int base = 0; base < nit; base += kGramRing) {
#pragma unroll
    for (int r0 = 0; r0 < kGramRing; r0 += CPI) {
#pragma unroll
      for (int q = 0; q < CPI; ++q) {
        stage(((r0 / CPI) & 1) * CPI + q, R[r0 + q]);
        load_chunk(base + r0 + q + kGramRing, R[r0 + q]);
      }
      lds_barrier();
#pragma unroll
      for (int q = 0; q < CPI; ++q) {
        const int r = ((r0 / CPI) & 1) * CPI + q;   // LDS buffer of this chunk
        const int c = base + r0 + q;
        if (c < nch) {
          if constexpr (FP8) {
            const unsigned char* kt = smem + (size_t)r * 2 * Sh::tile_bytes;
            const unsigned char* vt = kt + 32 * Sh::RS8;
            u32x2 X[NB], Y[NB];
            static_for<NB>([&](auto jc) {
              constexpr int j = decltype(jc)::value;
              if constexpr ((XM >> j) & 1u) X[j] = frag8(kt, j);
              if constexpr ((YM >> j) & 1u) Y[j] = frag8(vt, j);
            });
            static_for<NMB>([&](auto ic) {
              constexpr int i = decltype(ic)::value, b = B0 + i;
              if constexpr (b < NBB) {
                acc[i] = mfma_fp8(X[b % NB], Y[b / NB], acc[i]);
              } else {
                constexpr int k = b - NBB;
                acc[i] = mfma_fp8(X[gblk_col(k)], X[gblk_row(k)], acc[i]);
              }
            });
          } else {
            const uint16_t* kt = (const uint16_t*)(smem + (size_t)r * 2 * Sh::tile_bytes);
            const uint16_t* vt = kt + 32 * RS;
            u32x4 X[NB], Y[NB];
            static_for<NB>([&](auto jc) {
              constexpr int j = decltype(jc)::value;
              if constexpr ((XM >> j) & 1u) X[j] = frag(kt, j);
              if constexpr ((YM >> j) & 1u) Y[j] = frag(vt, j);
            });
            static_for<NMB>([&](auto ic) {
              constexpr int i = decltype(ic)::value, b = B0 + i;
              if constexpr (b < NBB) {
                acc[i] = mfma_bf16(X[b % NB], Y[b / NB], acc[i]);
              } else {
                constexpr int k = b - NBB;
                acc[i] = mfma_bf16(X[gblk_col(k)], X[gblk_row(k)], acc[i]);
              }
            });
          }
        }
      }
    }
  }

  // B blocks in accumulator layout scaled by c; G blocks (I, L), I >= L,
  // scaled by c^2: lane l = 16g + b owns row b, columns 4g..4g+3 of the block
  // (the values of C(L, I)) at bytes 8l..8l+7.  Both are written with
  // non-temporal stores: the state pass reads them long after this kernel.
  const size_t fh = (size_t)bh * a.Tc + tl;
  unsigned char* gout = (unsigned char*)a.gfr + fh * Sh::g_frame_bytes;
  unsigned char* bout = (unsigned char*)a.bfr + fh * Sh::b_frame_bytes;
  const float c2 = a.kscale2, c1 = a.kscale;
  static_for<NMB>([&](auto ic) {
    constexpr int i = decltype(ic)::value, b = B0 + i;
    const f32x4 x = acc[i];
    if constexpr (b < NBB) {
      const u32x2 v = {pack_bf16(c1 * x[0], c1 * x[1]), pack_bf16(c1 * x[2], c1 * x[3])};
      __builtin_nontemporal_store(v, (u32x2*)(bout + (size_t)b * 512 + l * 8));
    } else {
      const u32x2 v = {pack_bf16(c2 * x[0], c2 * x[1]), pack_bf16(c2 * x[2], c2 * x[3])};
      __builtin_nontemporal_store(v, (u32x2*)(gout + (size_t)(b - NBB) * 512 + l * 8));
    }
  });
}

template <int D, bool FP8, int NW, int CPI = 1>
__global__ __launch_bounds__(NW * 64, NW > GramShape<D>::NW ? 1 : 2) void gdn_gram_kernel(GramArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int fh = blockIdx.x;   // over BH * Tc
  const int bh = fh / a.Tc, tl = fh % a.Tc;
  // Workgroups past the last frame copy one head's state each (only the
  // short launches, with more waves than the default shape, are given a
  // copy): they run on CUs that the frames leave idle.
  constexpr bool kCanCopy = NW > GramShape<D>::NW;
  if (kCanCopy && fh >= a.BH * a.Tc) {
    constexpr int TH = NW * 64, PER = (D * D + TH - 1) / TH;
    const int h = fh - a.BH * a.Tc;
    const float* src = a.copy_src + (size_t)h * D * D;
    float* dst = a.copy_dst + (size_t)h * D * D;
    float x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = (int)threadIdx.x + i * TH;
      x[i] = u < D * D ? src[u] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = (int)threadIdx.x + i * TH;
      if (u < D * D) dst[u] = x[i];
    }
    return;
  }
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  static_for<NW>([&](auto wc) {
    constexpr int W = decltype(wc)::value;
    if (w == W) gram_wave<D, FP8, NW, W, CPI>(a, smem, bh, tl);
  });
}

// ----------------------------------------------------------------------------
// Gram pass, streaming form (used when a frame has enough chunks, see
// gram_stream_ok).  A persistent workgroup walks the (head, frame) pairs
// fh = wg, wg + G, ... of the launch, and all their chunks as one sequence, so
// the K/V prefetch runs across frame boundaries.  A finished frame's G and B
// go to an LDS staging buffer; during the next frame each wave copies one
// 1 KB piece of it to HBM per chunk.  Loads and stores share one in-order
// counter per wave: a load issued after a store can only be waited for once
// that store is done, so the stores are kept small, spread out and at least
// kGramRing chunks ahead of any load that is waited for -- writing a whole
// frame's output at once (the per-frame kernel above) stalls the load stream
// behind it.  The loop is branch-free except for the compute of real chunks
// and the frame-end staging, which hold no global memory operations.
// ----------------------------------------------------------------------------
template <int D>
struct GramStream {
  using Sh = GramShape<D>;
  static constexpr int GB = Sh::NBLK * 512;                  // G bytes per frame-head
  static constexpr int BB = Sh::NBB * 512;                   // B bytes per frame-head
  static constexpr int NGG = (GB + 1023) / 1024;             // 1 KB pieces of G
  static constexpr int NGB = (BB + 1023) / 1024;             // 1 KB pieces of B
  static constexpr int NP = NGG + NGB;                       // pieces per frame-head
  static constexpr size_t stage_off = Sh::lds_bytes;         // after the K/V tiles
  static constexpr size_t lds_bytes = stage_off + (size_t)NP * 1024;
};

// The staging buffer of a frame is fully copied out within ceil(NP/NW) chunks
// of the next frame, and a barrier must separate the last copy from the next
// frame-end staging.
template <int D>
constexpr int gram_stream_min_chunks() {
  return (GramStream<D>::NP + GramShape<D>::NW - 1) / GramShape<D>::NW + 1;
}
// ... and two workgroups must fit a CU's 160 KB of LDS (the per-frame kernel
// serves the head dims where they do not).
template <int D>
constexpr bool gram_stream_fits() {
  return 2 * GramStream<D>::lds_bytes <= 160 * 1024;
}

template <int D, bool FP8, int W>
__device__ __forceinline__ void gram_stream_wave(const GramArgs& a, unsigned char* smem) {
  using Sh = GramShape<D>;
  using St = GramStream<D>;
  using IO = IoFmt<FP8>;
  using raw = typename IO::raw;
  constexpr int NB = Sh::NB, NW = Sh::NW, UPR = Sh::UPR, NLD = Sh::NLD, LPW = Sh::LPW, RS = Sh::RS;
  constexpr int NBB = Sh::NBB, NOUT = Sh::NOUT, NGG = St::NGG, NP = St::NP;
  constexpr int B0 = W * NOUT / NW, B1 = (W + 1) * NOUT / NW, NMB = B1 - B0;   // my output blocks
  constexpr uint32_t XM = gram_xmask(NB, B0, B1), YM = gram_ymask(NB, B0, B1);
  const int l = lane_id(), g = l >> 4, n = l & 15;
  const int S = a.S, T = a.T, Tc = a.Tc;
  const int G = (int)gridDim.x, wg = (int)blockIdx.x, nfh = a.BH * Tc;
  const int nmine = wg < nfh ? (nfh - wg + G - 1) / G : 0;
  const int nch = (S + 31) / 32;
  const int total = nmine * nch;
  const int nit = (total + kGramRing - 1) / kGramRing * kGramRing;
  const uint32_t frame_bytes = (uint32_t)S * D * IO::ebytes;
  unsigned char* stage_buf = smem + St::stage_off;

  // Uniform conditions that decide whether a memory operation is real are
  // taken through a vector register, so that they become per-lane offset
  // selects instead of branches around the memory operation (a branch around
  // a load or store would make the compiler drain the whole counter).
  auto vgpr = [](int x) {
    asm volatile("" : "+v"(x));
    return x;
  };
  int lk = 0, lch = 0;   // next chunk to load: frame lk of this workgroup, chunk lch
  auto load_next = [&](raw (&X)[LPW]) {
    const int kk = lk < nmine ? lk : nmine - 1;          // a valid frame for the addresses
    const bool valid = vgpr(lk) < nmine;
    const int fh = wg + kk * G, bh = fh / Tc, tl = fh - bh * Tc;
    const size_t fe = ((size_t)bh * T + a.t0 + tl) * (size_t)S * D * IO::ebytes;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc((const unsigned char*)a.k + fe, frame_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const unsigned char*)a.v + fe, frame_bytes);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int p = W + NW * i;
      const int u = 64 * (p % NLD) + l;
      const int tok = lch * 32 + u / UPR;
      const bool ok = valid && p < 2 * NLD && tok < S;
      // offset past the buffer when !ok, by arithmetic (no select to branch on)
      const uint32_t off = (uint32_t)(lch * 32 * UPR + u) * IO::unit_bytes | ((uint32_t)!ok << 31);
      X[i] = IO::load_nt(p < NLD ? krs : vrs, off);
    }
    const bool wrap = lch + 1 == nch;
    lch = wrap ? 0 : lch + 1;
    lk += wrap ? 1 : 0;
  };
  // bf16 I/O: staged as bf16 (K through ReLU), bf16 MFMAs; e4m3 I/O:
  // staged as e4m3 codes, e4m3 MFMAs on the exact codes
  auto stage = [&](int buf, const raw (&X)[LPW]) {
    if constexpr (FP8) {
      unsigned char* kt = smem + (size_t)buf * 2 * Sh::tile_bytes;
      unsigned char* vt = kt + 32 * Sh::RS8;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int p = W + NW * i;
        if (p < 2 * NLD) {
          const int u = 64 * (p % NLD) + l;
          unsigned char* dst = (p < NLD ? kt : vt) + (u / UPR) * Sh::RS8 + 8 * (u % UPR);
          *(u32x2*)dst = p < NLD ? relu_e4m3x8(X[i]) : X[i];
        }
      }
    } else {
      uint16_t* kt = (uint16_t*)(smem + (size_t)buf * 2 * Sh::tile_bytes);
      uint16_t* vt = kt + 32 * RS;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int p = W + NW * i;
        if (p < 2 * NLD) {
          const int u = 64 * (p % NLD) + l;
          uint16_t* dst = (p < NLD ? kt : vt) + (u / UPR) * RS + 8 * (u % UPR);
          const u32x4 x = IO::to_bf16(X[i]);
          *(u32x4*)dst = p < NLD ? relu8(x) : x;
        }
      }
    }
  };
  auto frag = [&](const uint16_t* tile, int blk) -> u32x4 {
    const uint16_t* p0 = tile + (4 * g + (n >> 2)) * RS + 16 * blk + 4 * (n & 3);
    const u32x2 x = lds_tr16(p0), y = lds_tr16(p0 + 16 * RS);
    return u32x4{x[0], x[1], y[0], y[1]};
  };
  // e4m3 operand of block blk: lane l gets dim 16 blk + l % 16 of tokens
  // 8 (l / 16) .. + 7, the 16 lanes of a group naming rows (token, 8-byte
  // half) for the transposing read
  auto frag8 = [&](const unsigned char* tile, int blk) -> u32x2 {
    return lds_tr8(tile + (8 * g + (n >> 1)) * Sh::RS8 + 16 * blk + 8 * (n & 1));
  };
  // copy piece p of the staged frame k to its place in HBM (out-of-range
  // lanes, pieces and frames go to an offset past the buffer: no branch)
  auto store_piece = [&](int k, int p) {
    const int pp = p < NP ? p : 0;
    const int kk = k < 0 ? 0 : (k < nmine ? k : nmine - 1);
    const int kv = vgpr(k), pv = vgpr(p);
    const bool valid = kv >= 0 && kv < nmine && pv < NP;
    const u32x4 v = *(const u32x4*)(stage_buf + (size_t)pp * 1024 + l * 16);
    const size_t fh = (size_t)wg + (size_t)kk * G;
    const bool isg = pp < NGG;
    const __amdgpu_buffer_rsrc_t ors =
        isg ? make_rsrc((unsigned char*)a.gfr + fh * Sh::g_frame_bytes, (uint32_t)St::GB)
            : make_rsrc((unsigned char*)a.bfr + fh * Sh::b_frame_bytes, (uint32_t)St::BB);
    const uint32_t off = (uint32_t)((isg ? pp : pp - NGG) * 1024 + l * 16);
    __builtin_amdgcn_raw_buffer_store_b128(v, ors, valid ? off : kOOB, 0, kNT);
  };
  const float c2 = a.kscale2, c1 = a.kscale;

  f32x4 acc[NMB];
#pragma unroll
  for (int i = 0; i < NMB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  raw R[kGramRing][LPW];
#pragma unroll
  for (int r = 0; r < kGramRing; ++r) load_next(R[r]);

  int ck = 0, cch = 0;   // chunk being computed: frame ck of this workgroup, chunk cch
  for (int base = 0; base < nit; base += kGramRing) {
#pragma unroll
    for (int r = 0; r < kGramRing; ++r) {
      const int q = base + r;
      stage(r & 1, R[r]);
      load_next(R[r]);
      lds_barrier();
      // the previous frame's output, one piece per wave and chunk
      store_piece(ck - 1, cch * NW + W);
      if (q < total) {
        if constexpr (FP8) {
          const unsigned char* kt = smem + (size_t)(r & 1) * 2 * Sh::tile_bytes;
          const unsigned char* vt = kt + 32 * Sh::RS8;
          u32x2 X[NB], Y[NB];
          static_for<NB>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr ((XM >> j) & 1u) X[j] = frag8(kt, j);
            if constexpr ((YM >> j) & 1u) Y[j] = frag8(vt, j);
          });
          static_for<NMB>([&](auto ic) {
            constexpr int i = decltype(ic)::value, b = B0 + i;
            if constexpr (b < NBB) {
              acc[i] = mfma_fp8(X[b % NB], Y[b / NB], acc[i]);
            } else {
              constexpr int k = b - NBB;
              acc[i] = mfma_fp8(X[gblk_col(k)], X[gblk_row(k)], acc[i]);
            }
          });
        } else {
          const uint16_t* kt = (const uint16_t*)(smem + (size_t)(r & 1) * 2 * Sh::tile_bytes);
          const uint16_t* vt = kt + 32 * RS;
          u32x4 X[NB], Y[NB];
          static_for<NB>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr ((XM >> j) & 1u) X[j] = frag(kt, j);
            if constexpr ((YM >> j) & 1u) Y[j] = frag(vt, j);
          });
          static_for<NMB>([&](auto ic) {
            constexpr int i = decltype(ic)::value, b = B0 + i;
            if constexpr (b < NBB) {
              acc[i] = mfma_bf16(X[b % NB], Y[b / NB], acc[i]);
            } else {
              constexpr int k = b - NBB;
              acc[i] = mfma_bf16(X[gblk_col(k)], X[gblk_row(k)], acc[i]);
            }
          });
        }
        if (cch == nch - 1) {
          // frame complete: stage its blocks (B scaled by c, G by c^2, as in
          // the per-frame kernel) and start the next frame
          static_for<NMB>([&](auto ic) {
            constexpr int i = decltype(ic)::value, b = B0 + i;
            const f32x4 x = acc[i];
            const float cc = b < NBB ? c1 : c2;
            const u32x2 v = {pack_bf16(cc * x[0], cc * x[1]), pack_bf16(cc * x[2], cc * x[3])};
            const size_t so = b < NBB ? (size_t)NGG * 1024 + (size_t)b * 512 : (size_t)(b - NBB) * 512;
            *(u32x2*)(stage_buf + so + l * 8) = v;
            acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
          });
        }
        const bool wrap = cch + 1 == nch;
        cch = wrap ? 0 : cch + 1;
        ck += wrap ? 1 : 0;
      }
    }
  }
  // the last frame's output
  lds_barrier();
  for (int p = W; p < NP; p += NW) store_piece(nmine - 1, p);
}

template <int D, bool FP8>
__global__ __launch_bounds__(GramShape<D>::NW * 64, 2) void gdn_gram_stream_kernel(GramArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  static_for<GramShape<D>::NW>([&](auto wc) {
    constexpr int W = decltype(wc)::value;
    if (w == W) gram_stream_wave<D, FP8, W>(a, smem);
  });
}

// ----------------------------------------------------------------------------
// State pass.  One workgroup per (head, 16-wide value tile j), placed so that
// the tiles of a head share an XCD (they read the same G_t).  Wave I owns the
// 16 x 16 block M[16I..16I+15][16j..16j+15] in fp32 registers.  Per frame it
// forms (G_t bf16(M_{t-1}))[block I] with NKC MFMAs: the A operands come from
// the frame's stored G blocks, staged in LDS by all waves together (each G
// block is fetched once per workgroup), the B operands from the bf16 copy of
// the tile's state column that every wave published in LDS at the end of the
// previous frame.  Then the gate, the input term and the erase, the bf16
// publish and the snapshot store.  The global loads of G_t and B_t run
// kStateRing frames ahead in registers (they do not depend on the state); G
// moves from registers to its LDS slot one frame ahead of use.
// ----------------------------------------------------------------------------
constexpr int kStateRing = 6;   // even: the LDS buffers alternate with the frame parity

template <int D>
struct StateShape {
  static constexpr int NB = D / 16;
  static constexpr int NKC = (NB + 1) / 2;
  static constexpr int NGL = (int)(GramShape<D>::g_frame_bytes / 1024);   // 1 KB pieces of a frame's G
  static constexpr int LPG = (NGL + NB - 1) / NB;                        // pieces per wave
  static constexpr size_t g_slot = GramShape<D>::g_frame_bytes;
  // exchange slot (kb, lane): 16 bytes = blocks 2kb and 2kb+1 of that lane
  static constexpr size_t xch_bytes = (size_t)2 * NKC * 64 * 16;
  static constexpr size_t lds_bytes = 2 * g_slot + xch_bytes;
};

// Wave I of a state workgroup (I is a template parameter so that every block
// index below is a constant: which G blocks are read directly and which
// through a transposed read is fixed per wave, with no branches).
template <int D, bool ERASE, int I>
__device__ __forceinline__ void state_wave(const StateArgs& a, unsigned char* smem, int bh, int j) {
  using Sh = StateShape<D>;
  constexpr int NB = Sh::NB, NKC = Sh::NKC, NGL = Sh::NGL, LPG = Sh::LPG;
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, n = l & 15;
  const int Tc = a.Tc;
  unsigned char* gsl = smem;                                  // 2 G slots
  unsigned char* xch = smem + 2 * Sh::g_slot;                 // 2 exchange buffers
  (void)tid;

  // block NB of an odd block count is a zero pad of the last k-step
  if ((NB & 1) && I == 0) {
    *(u32x2*)(xch + ((size_t)(NKC - 1) * 64 + l) * 16 + 8) = u32x2{0u, 0u};
    *(u32x2*)(xch + Sh::xch_bytes / 2 + ((size_t)(NKC - 1) * 64 + l) * 16 + 8) = u32x2{0u, 0u};
  }

  const int row0 = 16 * I + 4 * g, col = 16 * j + n;
  f32x4 m = {0.f, 0.f, 0.f, 0.f};
  if (a.state_src) {
    const float* src = a.state_src + (size_t)bh * D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) m[r] = src[(size_t)(row0 + r) * D + col];
  }
  auto publish = [&](int buf, f32x4 x) {
    const u32x2 v = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
    *(u32x2*)(xch + (size_t)buf * (Sh::xch_bytes / 2) + ((size_t)(I >> 1) * 64 + l) * 16 + 8 * (I & 1)) = v;
    return v;
  };
  publish(0, m);

  const size_t gfb = GramShape<D>::g_frame_bytes, bfb = GramShape<D>::b_frame_bytes;
  // per-head buffer resources over this launch's frames of the staging
  // arrays ([head][Fs] frames, this launch from frame f0): < 2^31 bytes each
  const size_t fb = (size_t)bh * a.Fs + a.f0;
  const __amdgpu_buffer_rsrc_t grs = make_rsrc((const unsigned char*)a.gfr + fb * gfb, (uint32_t)(Tc * gfb));
  const __amdgpu_buffer_rsrc_t brs = make_rsrc((const unsigned char*)a.bfr + fb * bfb, (uint32_t)(Tc * bfb));
  const size_t sfb = (size_t)bh * a.snap_Fs + a.snap_f0;
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc((unsigned char*)a.snap + sfb * D * D * 2, (uint32_t)(Tc * D * D * 2));
  const __amdgpu_buffer_rsrc_t gars = make_rsrc(a.gamma + (size_t)bh * a.T + a.t0, (uint32_t)(Tc * 4));
  const __amdgpu_buffer_rsrc_t bers = make_rsrc(a.beta + (size_t)bh * a.T + a.t0, (uint32_t)(Tc * 4));
  const uint32_t bbase = (uint32_t)((j * NB + I) * 512 + l * 8);
  const uint32_t sbase = (uint32_t)(((j * NB + I) * 64 + l) * 8);

  u32x4 Gr[kStateRing][LPG];                  // this wave's 1 KB pieces of a frame's G
  u32x2 Bf[kStateRing];
  float Ga[kStateRing], Be[kStateRing];       // gamma_t, beta_t
  auto load_frame = [&](int f, int r) {
    const bool ok = f < Tc;
    Ga[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gars, ok ? (uint32_t)f * 4u : kOOB, 0, 0));
    Be[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(bers, ok ? (uint32_t)f * 4u : kOOB, 0, 0));
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      const int q = I + NB * i;             // piece index (uniform)
      Gr[r][i] = buf_load16(grs, (ok && q < NGL) ? (uint32_t)f * (uint32_t)gfb + q * 1024 + l * 16 : kOOB);
    }
    Bf[r] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                          brs, ok ? bbase + (uint32_t)f * (uint32_t)bfb : kOOB, 0, kNT));
  };
  auto stage_g = [&](int slot, int r) {
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      const int q = I + NB * i;
      if (q < NGL) *(u32x4*)(gsl + (size_t)slot * Sh::g_slot + q * 1024 + l * 16) = Gr[r][i];
    }
  };
  // A operand half: row a = n of block (I, L), columns 4g..4g+3
  auto g_half = [&](const unsigned char* gs, auto Lc) -> u32x2 {
    constexpr int L = decltype(Lc)::value;
    if constexpr (L >= NB) {
      return u32x2{0u, 0u};
    } else if constexpr (L <= I) {
      return *(const u32x2*)(gs + (size_t)(I * (I + 1) / 2 + L) * 512 + l * 8);
    } else {
      // block (I, L) = transpose of the stored block (L, I): column n of its
      // rows 4g..4g+3, through a transposed read in which lane j of the
      // 16-lane group supplies row 4g + j/4, columns 4(j%4)..+3
      const unsigned char* blk = gs + (size_t)(L * (L + 1) / 2 + I) * 512;
      return lds_tr16((const uint16_t*)(blk + ((n & 3) * 16 + 4 * g + (n >> 2)) * 8));
    }
  };

#pragma unroll
  for (int r = 0; r < kStateRing; ++r) load_frame(r, r);
  stage_g(0, 0);
  lds_barrier();

  for (int base = 0; base < Tc; base += kStateRing) {
#pragma unroll
    for (int r = 0; r < kStateRing; ++r) {
      const int f = base + r;
      const unsigned char* xr = xch + (size_t)(r & 1) * (Sh::xch_bytes / 2);
      const unsigned char* gs = gsl + (size_t)(r & 1) * Sh::g_slot;
      // all operand reads first (one LDS latency per frame), then the MFMA chain
      u32x4 aop[NKC], bop[NKC];
      static_for<NKC>([&](auto kbc) {
        constexpr int kb = decltype(kbc)::value;
        const u32x2 lo = g_half(gs, Int<2 * kb>{}), hi = g_half(gs, Int<2 * kb + 1>{});
        aop[kb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        bop[kb] = *(const u32x4*)(xr + ((size_t)kb * 64 + l) * 16);
      });
      __builtin_amdgcn_sched_barrier(0);
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) p = mfma_bf16(aop[kb], bop[kb], p);
      const float gm = Ga[r], bt = Be[r], bg = bt * gm;
      const u32x2 bw = Bf[r];
      const f32x4 bin = {bf16_lo_f32(bw[0]), bf16_hi_f32(bw[0]), bf16_lo_f32(bw[1]), bf16_hi_f32(bw[1])};
      const bool ok = f < Tc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float nv = state_update(gm, m[e], bg, p[e], ERASE ? bin[e] : bt * bin[e]);
        m[e] = ok ? nv : m[e];
      }
      // G of the next frame into the other LDS slot (read by everyone after the barrier)
      stage_g((r + 1) & 1, (r + 1) % kStateRing);
      load_frame(f + kStateRing, r);
      const u32x2 pub = publish((r & 1) ^ 1, m);
      // bf16 snapshot of M_t: this wave's block, lane-linear (512 contiguous bytes)
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pub), srs,
                                            ok ? sbase + (uint32_t)f * (uint32_t)(D * D * 2) : kOOB, 0, 0);
      lds_barrier();
    }
  }

  if (a.state_dst) {
    float* dst = a.state_dst + (size_t)bh * D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(size_t)(row0 + r) * D + col] = m[r];
  }
}

template <int D, bool ERASE>
__global__ __launch_bounds__(D / 16 * 64, 1) void gdn_state_bf16_kernel(StateArgs a) {
  constexpr int NB = D / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int unit = xcd_unit(a.BH * NB);
  if (unit < 0) return;                       // whole workgroup: no work on this slot
  const int bh = unit / NB, j = unit % NB;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  static_for<NB>([&](auto ic) {
    constexpr int I = decltype(ic)::value;
    if (w == I) state_wave<D, ERASE, I>(a, smem, bh, j);
  });
}


// ----------------------------------------------------------------------------
// Chunk tail: the state chain and the readout of a short launch (a streaming
// chunk of at most kTailMaxFrames frames per head) in one kernel.  There the
// serial state pass and a readout launch behind it cost far more than the
// chain itself.  One workgroup per (head, frame t, share of the frame's
// token chunks), NB waves.  Wave I owns key-block row I of the state for
// every value tile j and first runs the chain over the launch's frames
// 0..t: per element the same instructions as gdn_state_bf16_kernel (the
// product over the G row and the bf16 state column of tile j, then the
// gate, input and erase), hence the same bits.  That leaves bf16(M_t) in
// LDS exactly as the readout's A operands.  Then the waves read out
// O_t = ReLU(Q_t) M_t for their chunks with the readout kernel's MFMA order
// (the same bits as gdn_readout_kernel), each lane storing its 4
// consecutive output columns of every value tile.  A workgroup recomputes
// the frames before its own instead of waiting for another workgroup, so no
// workgroup ever waits on another, and Q is read once.  All frames' G and B
// are loaded first, then the first Q chunks, which stay in flight during
// the chain.  The workgroup of the last frame (share 0) writes the fp32
// state; state_src is read by every workgroup and so must not alias
// state_dst (the caller passes a copy).
// ----------------------------------------------------------------------------
template <int D>
struct TailShape {
  using St = StateShape<D>;
  static constexpr int NB = D / 16, NKC = St::NKC;
  static constexpr int UPR = D / 8, NLD = D / 16, RS = D + 8;
  static constexpr int QRING = D >= 80 ? 2 : 3;       // Q chunks in flight per wave
  static constexpr int FRING = kTailMaxFrames;        // frames of G, B, gamma, beta (all of them)
  // exchange buffer: per value tile j the state kernel's slots (kb, lane)
  static constexpr size_t xtile = (size_t)NKC * 64 * 16;
  static constexpr size_t xbuf = NB * xtile;
  static constexpr size_t xch_off = 2 * St::g_slot;
  static constexpr size_t qtile_off = xch_off + 2 * xbuf;
  static constexpr size_t qtile_bytes = (size_t)32 * RS * 2;
  static constexpr size_t lds_bytes = qtile_off + (size_t)NB * qtile_bytes;
};
constexpr bool tail_fits(int D) { return D <= 112; }   // LDS (D = 128 would need 170 KB)

template <int D, bool FP8, bool ERASE, int I>
__device__ __forceinline__ void tail_wave(const TailArgs& a, unsigned char* smem, int bh, int tl, int sp) {
  using Sh = StateShape<D>;
  using Tl = TailShape<D>;
  using IO = IoFmt<FP8>;
  using raw = typename IO::raw;
  constexpr int NB = Sh::NB, NKC = Sh::NKC, NGL = Sh::NGL, LPG = Sh::LPG;
  constexpr int UPR = Tl::UPR, NLD = Tl::NLD, RS = Tl::RS, FR = Tl::FRING;
  // e4m3 at D >= 96 keeps one chunk in flight (the conversions' registers)
  constexpr int QR = FP8 && D >= 96 ? 1 : Tl::QRING;
  const int l = lane_id(), g = l >> 4, n = l & 15;
  unsigned char* gsl = smem;                                  // 2 G slots
  unsigned char* xch = smem + Tl::xch_off;                    // 2 exchange buffers
  uint16_t* qs = (uint16_t*)(smem + Tl::qtile_off + (size_t)I * Tl::qtile_bytes);
  const int S = a.S, T = a.T, t = a.t0 + tl;

  // ---- Q chunks of this wave: chunk wt + RWT i of the frame ----
  const uint32_t head_bytes = (uint32_t)T * (uint32_t)S * D * IO::ebytes;
  const size_t head0 = (size_t)bh * T * S * D * IO::ebytes;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc((const unsigned char*)a.q + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t ors = make_rsrc((unsigned char*)a.o + head0, head_bytes);
  const uint32_t fbyte = (uint32_t)t * (uint32_t)S * D * IO::ebytes;
  const int nchunk = (S + 31) / 32;
  const int RWT = NB * a.nsplit, wt = NB * sp + I;
  const int NC = (nchunk + RWT - 1) / RWT;
  auto unit_off = [&](int ch, int u) -> uint32_t {
    const int tok = ch * 32 + u / UPR;
    return (ch < nchunk && tok < S) ? fbyte + (uint32_t)(ch * 32 * UPR + u) * IO::unit_bytes : kOOB;
  };
  auto load_chunk = [&](int i, raw (&X)[NLD]) {
    const int ch = wt + RWT * i;
#pragma unroll
    for (int u = 0; u < NLD; ++u) X[u] = IO::load_nt(qrs, i < NC ? unit_off(ch, 64 * u + l) : kOOB);
  };
  raw X[QR][NLD];

  // ---- the chain over frames 0..tl: block (I, j) of every tile j ----
  if ((NB & 1) && I == 0) {
    // block NB of an odd block count is a zero pad of the last k-step
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      *(u32x2*)(xch + j * Tl::xtile + ((size_t)(NKC - 1) * 64 + l) * 16 + 8) = u32x2{0u, 0u};
      *(u32x2*)(xch + Tl::xbuf + j * Tl::xtile + ((size_t)(NKC - 1) * 64 + l) * 16 + 8) = u32x2{0u, 0u};
    }
  }
  const int row0 = 16 * I + 4 * g;
  f32x4 m[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) m[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (a.state_src) {
    const float* src = a.state_src + (size_t)bh * D * D;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) m[j][r] = src[(size_t)(row0 + r) * D + 16 * j + n];
  }
  auto publish = [&](int buf, int j, f32x4 x) {
    const u32x2 v = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
    *(u32x2*)(xch + (size_t)buf * Tl::xbuf + j * Tl::xtile + ((size_t)(I >> 1) * 64 + l) * 16 + 8 * (I & 1)) = v;
  };
#pragma unroll
  for (int j = 0; j < NB; ++j) publish(0, j, m[j]);

  const int Tc = a.Tc;
  const size_t gfb = GramShape<D>::g_frame_bytes, bfb = GramShape<D>::b_frame_bytes;
  const size_t fb = (size_t)bh * Tc;
  const __amdgpu_buffer_rsrc_t grs = make_rsrc((const unsigned char*)a.gfr + fb * gfb, (uint32_t)(Tc * gfb));
  const __amdgpu_buffer_rsrc_t brs = make_rsrc((const unsigned char*)a.bfr + fb * bfb, (uint32_t)(Tc * bfb));
  const __amdgpu_buffer_rsrc_t gars = make_rsrc(a.gamma + (size_t)bh * T + a.t0, (uint32_t)(Tc * 4));
  const __amdgpu_buffer_rsrc_t bers = make_rsrc(a.beta + (size_t)bh * T + a.t0, (uint32_t)(Tc * 4));

  u32x4 Gr[FR][LPG];
  u32x2 Bf[FR][NB];                        // B blocks (j, I), lane-linear as the state pass reads them
  float Ga[FR], Be[FR];
  auto load_frame = [&](int f) {
    const bool ok = f <= tl;
    Ga[f] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gars, ok ? (uint32_t)f * 4u : kOOB, 0, 0));
    Be[f] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(bers, ok ? (uint32_t)f * 4u : kOOB, 0, 0));
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      const int q = I + NB * i;
      Gr[f][i] = buf_load16(grs, (ok && q < NGL) ? (uint32_t)f * (uint32_t)gfb + q * 1024 + l * 16 : kOOB);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
      Bf[f][j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                               brs, ok ? (uint32_t)((j * NB + I) * 512 + l * 8) + (uint32_t)f * (uint32_t)bfb
                                                       : kOOB, 0, 0));
  };
  auto stage_g = [&](int slot, int f) {
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      const int q = I + NB * i;
      if (q < NGL) *(u32x4*)(gsl + (size_t)slot * Sh::g_slot + q * 1024 + l * 16) = Gr[f][i];
    }
  };
  auto g_half = [&](const unsigned char* gs, auto Lc) -> u32x2 {
    constexpr int L = decltype(Lc)::value;
    if constexpr (L >= NB) {
      return u32x2{0u, 0u};
    } else if constexpr (L <= I) {
      return *(const u32x2*)(gs + (size_t)(I * (I + 1) / 2 + L) * 512 + l * 8);
    } else {
      const unsigned char* blk = gs + (size_t)(L * (L + 1) / 2 + I) * 512;
      return lds_tr16((const uint16_t*)(blk + ((n & 3) * 16 + 4 * g + (n >> 2)) * 8));
    }
  };

  // Every frame's G, B, gamma and beta, then the first Q chunks: the chain
  // below issues no load, so each of its waits is for exactly the frame
  // loads it needs (loads complete in issue order).
#pragma unroll
  for (int f = 0; f < FR; ++f) load_frame(f);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < QR; ++r) load_chunk(r, X[r]);
  __builtin_amdgcn_sched_barrier(0);
  stage_g(0, 0);
  lds_barrier();
  // All FR frames, unrolled; those past tl are computed on zeros and not
  // committed, so no branch splits the waits.
#pragma unroll
  for (int f = 0; f < FR; ++f) {
    __builtin_amdgcn_sched_barrier(0);       // no work of a later frame moves up (its waits would follow)
    const bool ok = f <= tl;
    const unsigned char* xr = xch + (size_t)(f & 1) * Tl::xbuf;
    const unsigned char* gs = gsl + (size_t)(f & 1) * Sh::g_slot;
    u32x4 aop[NKC];
    static_for<NKC>([&](auto kbc) {
      constexpr int kb = decltype(kbc)::value;
      const u32x2 lo = g_half(gs, Int<2 * kb>{}), hi = g_half(gs, Int<2 * kb + 1>{});
      aop[kb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    });
    const float gm = Ga[f], bt = Be[f], bg = bt * gm;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      u32x4 bop[NKC];
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) bop[kb] = *(const u32x4*)(xr + j * Tl::xtile + ((size_t)kb * 64 + l) * 16);
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) p = mfma_bf16(aop[kb], bop[kb], p);
      const u32x2 bw = Bf[f][j];
      const f32x4 bin = {bf16_lo_f32(bw[0]), bf16_hi_f32(bw[0]), bf16_lo_f32(bw[1]), bf16_hi_f32(bw[1])};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float nv = state_update(gm, m[j][e], bg, p[e], ERASE ? bin[e] : bt * bin[e]);
        m[j][e] = ok ? nv : m[j][e];
      }
    }
    if (f + 1 < FR) stage_g((f + 1) & 1, f + 1);
#pragma unroll
    for (int j = 0; j < NB; ++j) publish((f & 1) ^ 1, j, m[j]);
    lds_barrier();
  }
  if (tl == Tc - 1 && sp == 0 && a.state_dst) {
    float* dst = a.state_dst + (size_t)bh * D * D;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(row0 + r) * D + 16 * j + n] = m[j][r];
  }

  // ---- readout: A operand (jb, kc) = exchange slot (jb, kc) of bf16(M_t) ----
  const unsigned char* xf = xch + (size_t)(FR & 1) * Tl::xbuf;   // published after frame FR - 1
  u32x4 A[NB][NKC];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb)
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) A[jb][kc] = *(const u32x4*)(xf + jb * Tl::xtile + ((size_t)kc * 64 + l) * 16);
  for (int base = 0; base < NC; base += QR) {
#pragma unroll
    for (int r = 0; r < QR; ++r) {
      const int i = base + r;
      const int ch = wt + RWT * i;
      // Nothing of a later slot moves up: the compiler would hoist the ReLU
      // of the next chunks and with it the waits for their loads.
      __builtin_amdgcn_sched_barrier(0);
      // branch-free like the chain: a slot past the wave's last chunk reads
      // zeros and its stores are dropped (chunk index past the frame)
#pragma unroll
      for (int u = 0; u < NLD; ++u) {
        const int uu = 64 * u + l;
        *(u32x4*)(qs + (uu / UPR) * RS + 8 * (uu % UPR)) = relu8(IO::to_bf16(X[r][u]));
      }
      load_chunk(i + QR, X[r]);
      wave_lds_sync();
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 B[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          const uint16_t* rp = qs + (16 * half + n) * RS + 32 * kc + 4 * g;
          const u32x2 lo = *(const u32x2*)rp;
          const u32x2 hi = (32 * kc + 32 <= D) ? *(const u32x2*)(rp + 16) : u32x2{0u, 0u};
          B[kc] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
        const int tok = ch * 32 + 16 * half + n;
        const bool in = ch < nchunk && tok < S;
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) acc = mfma_bf16(A[jb][kc], B[kc], acc);
          const uint32_t off = in ? fbyte + ((uint32_t)tok * D + 16 * jb + 4 * g) * IO::ebytes : kOOB;
          if constexpr (FP8) {
            __builtin_amdgcn_raw_buffer_store_b32(f32x4_to_fp8x4(acc), ors, off, 0, 0);
          } else {
            const u32x2 pk = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
            __builtin_amdgcn_raw_buffer_store_b64(pk, ors, off, 0, 0);
          }
        }
      }
      wave_lds_sync();
    }
  }
}

template <int D, bool FP8, bool ERASE>
__global__ __launch_bounds__(D / 16 * 64) void gdn_step_tail_kernel(TailArgs a) {
  constexpr int NB = D / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if constexpr (tail_fits(D)) {
    const int nsp = a.nsplit;
    const int unit = xcd_unit(a.BH * a.Tc * nsp);
    if (unit < 0) return;                     // whole workgroup: no work on this slot
    const int sp = unit % nsp, fr = unit / nsp;
    const int bh = fr / a.Tc, tl = fr % a.Tc;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    static_for<NB>([&](auto ic) {
      constexpr int I = decltype(ic)::value;
      if (w == I) tail_wave<D, FP8, ERASE, I>(a, smem, bh, tl, sp);
    });
  }
}

// ----------------------------------------------------------------------------
// Backward: C_t = ReLU(Q_t)^T dO_t and dQ_t = (dO_t M_t^T) * [Q_t > 0] in one
// pass over Q_t and dO_t.  One workgroup per (head, frame) with the gram
// pass's waves and chunk pipeline (Q in the key's place, dO in the value's):
// every wave accumulates its compile-time range of the NB*NB blocks of C as
// the gram pass accumulates B, and also forms dQ for its output column
// blocks jb = W, W + NW, ... from the staged chunk, with M_t^T as MFMA A
// operands in registers (transposed LDS reads of the staged snapshot of
// M_t) and the mask read from the staged ReLU(Q).  dQ is assembled in an LDS
// tile and stored with the loads' coalesced 1 KB pieces; C goes out at the
// end of the frame in B's layout.
// ----------------------------------------------------------------------------
template <int D, int W>
__device__ __forceinline__ void cdq_wave(const CdqArgs& a, unsigned char* smem, int bh, int t) {
  using Sh = GramShape<D>;
  constexpr int NB = Sh::NB, NW = Sh::NW, UPR = Sh::UPR, NLD = Sh::NLD, LPW = Sh::LPW, RS = Sh::RS;
  constexpr int NKC = Sh::NKC, NBB = Sh::NBB;
  constexpr int B0 = W * NBB / NW, B1 = (W + 1) * NBB / NW, NMB = B1 - B0;   // my C blocks
  constexpr uint32_t XM = gram_xmask(NB, B0, B1), YM = gram_ymask(NB, B0, B1);
  constexpr int JPW = (NB + NW - 1) / NW;                                    // my dQ column blocks
  constexpr int SPW = (NLD + NW - 1) / NW;                                   // dQ pieces stored per wave
  const int l = lane_id(), g = l >> 4, n = l & 15;
  const int S = a.S, T = a.T;
  const uint32_t head_bytes = (uint32_t)T * (uint32_t)S * D * 2u;
  const size_t head0 = (size_t)bh * T * S * D * 2;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc((const unsigned char*)a.q + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc((const unsigned char*)a.dout + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t dqrs =
      make_rsrc(a.dq ? (unsigned char*)a.dq + head0 : nullptr, a.dq ? head_bytes : 0u);
  const uint32_t fbyte = (uint32_t)t * (uint32_t)S * D * 2u;
  // chunks in flight (even, for the LDS buffer parity); at D = 128 a deeper
  // ring does not fit the registers next to the C accumulators and M_t^T
  constexpr int RG = D >= 128 ? 2 : kGramRing;
  const int nch = (S + 31) / 32;
  const int nit = (nch + RG - 1) / RG * RG;
  uint16_t* const ot = (uint16_t*)(smem + 4 * Sh::tile_bytes);               // dQ tile

  // M_t^T operands of my column blocks (snapshot staged in the tiles' space)
  const unsigned char* msn = (const unsigned char*)a.msnap + ((size_t)bh * (T + 1) + t + 1) * D * D * 2;
  for (int u = (int)threadIdx.x; u < D * D * 2 / 16; u += NW * 64)
    *(u32x4*)(smem + (size_t)u * 16) = *(const u32x4*)(msn + (size_t)u * 16);
  __syncthreads();
  const uint32_t trofs = (uint32_t)(((n & 3) * 16 + 4 * g + (n >> 2)) * 8);
  u32x4 AM[JPW][NKC];
  static_for<JPW>([&](auto ic) {
    constexpr int i = decltype(ic)::value, jb = W + NW * i;
    if constexpr (jb < NB) {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const u32x2 lo = lds_tr16((const uint16_t*)(smem + (size_t)((2 * kc) * NB + jb) * 512 + trofs));
        const u32x2 hi = (2 * kc + 1 < NB)
                             ? lds_tr16((const uint16_t*)(smem + (size_t)((2 * kc + 1) * NB + jb) * 512 + trofs))
                             : u32x2{0u, 0u};
        AM[i][kc] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    }
  });
  __syncthreads();

  auto unit_off = [&](int ch, int u) -> uint32_t {
    const int tok = ch * 32 + u / UPR;
    return (ch < nch && tok < S) ? fbyte + (uint32_t)(ch * 32 * UPR + u) * 16u : kOOB;
  };
  auto load_chunk = [&](int ch, u32x4 (&X)[LPW]) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int p = W + NW * i;
      const uint32_t off = p < 2 * NLD ? unit_off(ch, 64 * (p % NLD) + l) : kOOB;
      X[i] = buf_load16_nt(p < NLD ? qrs : drs, off);
    }
  };
  auto stage = [&](int buf, const u32x4 (&X)[LPW]) {
    uint16_t* qt = (uint16_t*)(smem + (size_t)buf * 2 * Sh::tile_bytes);
    uint16_t* dt = qt + 32 * RS;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int p = W + NW * i;
      if (p < 2 * NLD) {
        const int u = 64 * (p % NLD) + l;
        *(u32x4*)((p < NLD ? qt : dt) + (u / UPR) * RS + 8 * (u % UPR)) = p < NLD ? relu8(X[i]) : X[i];
      }
    }
  };
  auto frag = [&](const uint16_t* tile, int blk) -> u32x4 {
    const uint16_t* p0 = tile + (4 * g + (n >> 2)) * RS + 16 * blk + 4 * (n & 3);
    const u32x2 x = lds_tr16(p0), y = lds_tr16(p0 + 16 * RS);
    return u32x4{x[0], x[1], y[0], y[1]};
  };

  f32x4 acc[NMB];
#pragma unroll
  for (int i = 0; i < NMB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 R[RG][LPW];
#pragma unroll
  for (int r = 0; r < RG; ++r) load_chunk(r, R[r]);

  for (int base = 0; base < nit; base += RG) {
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int c = base + r;
      stage(r & 1, R[r]);
      load_chunk(c + RG, R[r]);
      lds_barrier();
      if (c < nch) {
        const uint16_t* qt = (const uint16_t*)(smem + (size_t)(r & 1) * 2 * Sh::tile_bytes);
        const uint16_t* dt = qt + 32 * RS;
        u32x4 X[NB], Y[NB];
        static_for<NB>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          if constexpr ((XM >> j) & 1u) X[j] = frag(qt, j);
          if constexpr ((YM >> j) & 1u) Y[j] = frag(dt, j);
        });
        static_for<NMB>([&](auto ic) {
          constexpr int i = decltype(ic)::value, b = B0 + i;
          acc[i] = mfma_bf16(X[b % NB], Y[b / NB], acc[i]);
        });
        static_for<JPW>([&](auto ic) {
          constexpr int i = decltype(ic)::value, jb = W + NW * i;
          if constexpr (jb < NB) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              u32x4 BD[NKC];
#pragma unroll
              for (int kc = 0; kc < NKC; ++kc) {
                const uint16_t* rp = dt + (16 * half + n) * RS + 32 * kc + 4 * g;
                const u32x2 lo = *(const u32x2*)rp;
                const u32x2 hi = (32 * kc + 32 <= D) ? *(const u32x2*)(rp + 16) : u32x2{0u, 0u};
                BD[kc] = u32x4{lo[0], lo[1], hi[0], hi[1]};
              }
              f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int kc = 0; kc < NKC; ++kc) y = mfma_bf16(AM[i][kc], BD[kc], y);
              const int oo = (16 * half + n) * RS + 16 * jb + 4 * g;
              const u32x2 qr = *(const u32x2*)(qt + oo);    // ReLU(Q) at the same (token, column)
              y[0] = (qr[0] & 0xffffu) ? y[0] : 0.f;
              y[1] = (qr[0] >> 16) ? y[1] : 0.f;
              y[2] = (qr[1] & 0xffffu) ? y[2] : 0.f;
              y[3] = (qr[1] >> 16) ? y[3] : 0.f;
              *(u32x2*)(ot + oo) = u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
            }
          }
        });
      }
      lds_barrier();
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const int p = W + NW * i;
        if (p < NLD) {
          const int u = 64 * p + l;
          const u32x4 yv = *(const u32x4*)(ot + (u / UPR) * RS + 8 * (u % UPR));
          __builtin_amdgcn_raw_buffer_store_b128(yv, dqrs, unit_off(c, u), 0, kNT);
        }
      }
    }
  }
  // C blocks in B's layout (scale 1)
  unsigned char* cout = (unsigned char*)a.cfr + ((size_t)bh * T + t) * Sh::b_frame_bytes;
  static_for<NMB>([&](auto ic) {
    constexpr int i = decltype(ic)::value, b = B0 + i;
    const f32x4 x = acc[i];
    *(u32x2*)(cout + (size_t)b * 512 + l * 8) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
  });
}

template <int D>
__global__ __launch_bounds__(GramShape<D>::NW * 64, 2) void gdn_cdq_kernel(CdqArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int fh = blockIdx.x;   // over BH * Tc
  const int bh = fh / a.Tc, t = a.t0 + fh % a.Tc;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  static_for<GramShape<D>::NW>([&](auto wc) {
    constexpr int W = decltype(wc)::value;
    if (w == W) cdq_wave<D, W>(a, smem, bh, t);
  });
}

// ----------------------------------------------------------------------------
// Adjoint state pass (backward).  Write Lambda_t for dL/dM_t, the gradient of
// the loss with respect to the post-update state of frame t through
// everything after it.  The forward update M_t = g M_{t-1} - b g G_t M_{t-1} +
// w B_t (w = 1 ERASE, b WRITE) and the readout O_t = ReLU(Q_t) M_t give,
// frames last to first,
//   Lambda_{T-1} = dL/dM_final + C_{T-1},       C_t = ReLU(Q_t)^T dO_t,
//   Lambda_{t-1} = g_t Lambda_t - b_t g_t G_t Lambda_t + C_{t-1}
// (G_t is symmetric), and dL/dM_in = g_0 Lambda_0 - b_0 g_0 G_0 Lambda_0.  The
// workgroup layout is the state pass's: one workgroup per (head, value tile
// j), wave I owns the fp32 block Lambda[16I..16I+15][16j..16j+15], and the
// product G_t bf16(Lambda_t) is formed as the state pass forms G_t bf16(M).
// Per frame each wave also writes its block of the bf16 snapshot of Lambda_t
// and the partial sums over its block of <Lambda_t, M_{t-1}>,
// <G_t Lambda_t, M_{t-1}> and (WRITE) <Lambda_t, B_t>, from which
//   dL/dg_t = <Lambda_t, M_{t-1}> - b_t <G_t Lambda_t, M_{t-1}>,
//   dL/db_t = -g_t <G_t Lambda_t, M_{t-1}>   (+ <Lambda_t, B_t> for WRITE)
// are summed in a fixed order by gdn_adjoint_reduce.
// ----------------------------------------------------------------------------
template <int D, bool ERASE, int I>
__device__ __forceinline__ void adjoint_wave(const AdjointArgs& a, unsigned char* smem, int bh, int j) {
  using Sh = StateShape<D>;
  constexpr int NB = Sh::NB, NKC = Sh::NKC, NGL = Sh::NGL, LPG = Sh::LPG;
  const int l = lane_id(), g = l >> 4, n = l & 15;
  const int T = a.T;
  unsigned char* gsl = smem;                                  // 2 G slots
  unsigned char* xch = smem + 2 * Sh::g_slot;                 // 2 exchange buffers

  if ((NB & 1) && I == 0) {
    *(u32x2*)(xch + ((size_t)(NKC - 1) * 64 + l) * 16 + 8) = u32x2{0u, 0u};
    *(u32x2*)(xch + Sh::xch_bytes / 2 + ((size_t)(NKC - 1) * 64 + l) * 16 + 8) = u32x2{0u, 0u};
  }
  const int row0 = 16 * I + 4 * g, col = 16 * j + n;
  const size_t gfb = GramShape<D>::g_frame_bytes, bfb = GramShape<D>::b_frame_bytes;
  const size_t sfb = (size_t)D * D * 2;
  const size_t hb = (size_t)bh * T;
  const __amdgpu_buffer_rsrc_t grs = make_rsrc((const unsigned char*)a.gfr + hb * gfb, (uint32_t)(T * gfb));
  const __amdgpu_buffer_rsrc_t brs = make_rsrc((const unsigned char*)a.bfr + hb * bfb, (uint32_t)(T * bfb));
  const __amdgpu_buffer_rsrc_t crs = make_rsrc((const unsigned char*)a.cfr + hb * bfb, (uint32_t)(T * bfb));
  const __amdgpu_buffer_rsrc_t mrs =
      make_rsrc((const unsigned char*)a.msnap + (size_t)bh * (T + 1) * sfb, (uint32_t)((T + 1) * sfb));
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc((unsigned char*)a.lsnap + hb * sfb, (uint32_t)(T * sfb));
  const __amdgpu_buffer_rsrc_t prs =
      make_rsrc(a.part + hb * (size_t)(NB * NB * 4), (uint32_t)(T * NB * NB * 16));
  const __amdgpu_buffer_rsrc_t gars = make_rsrc(a.gamma + hb, (uint32_t)(T * 4));
  const __amdgpu_buffer_rsrc_t bers = make_rsrc(a.beta + hb, (uint32_t)(T * 4));
  const uint32_t bbase = (uint32_t)((j * NB + I) * 512 + l * 8);        // B / C block (I, j)
  const uint32_t sbase = (uint32_t)(((j * NB + I) * 64 + l) * 8);       // snapshot block (I, j)
  auto widen4 = [](u32x2 w) -> f32x4 {
    return f32x4{bf16_lo_f32(w[0]), bf16_hi_f32(w[0]), bf16_lo_f32(w[1]), bf16_hi_f32(w[1])};
  };

  // Lambda_{t_hi-1}: carried from the previous launch, or, for the first
  // launch (t_hi = T), dL/dM_final + C_{T-1}
  const int t_hi = a.t_hi, Tc = a.t_hi - a.t_lo;
  f32x4 m = {0.f, 0.f, 0.f, 0.f};
  if (a.lam_src) {
    const float* src = a.lam_src + (size_t)bh * D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) m[r] = src[(size_t)(row0 + r) * D + col];
  } else {
    if (a.dstate_out) {
      const float* src = a.dstate_out + (size_t)bh * D * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) m[r] = src[(size_t)(row0 + r) * D + col];
    }
    const f32x4 c0 = widen4(__builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(crs, (uint32_t)(T - 1) * (uint32_t)bfb + bbase, 0, 0)));
    m += c0;
  }
  auto publish = [&](int buf, f32x4 x) {
    const u32x2 v = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
    *(u32x2*)(xch + (size_t)buf * (Sh::xch_bytes / 2) + ((size_t)(I >> 1) * 64 + l) * 16 + 8 * (I & 1)) = v;
    return v;
  };
  u32x2 pub = publish(0, m);

  u32x4 Gr[kStateRing][LPG];
  u32x2 Cp[kStateRing], Mp[kStateRing], Bf[kStateRing];
  float Ga[kStateRing], Be[kStateRing];
  // step u handles frame t = t_hi-1-u
  auto load_frame = [&](int u, int r) {
    const int t = t_hi - 1 - u;
    const bool ok = u < Tc;
    Ga[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gars, ok ? (uint32_t)t * 4u : kOOB, 0, 0));
    Be[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(bers, ok ? (uint32_t)t * 4u : kOOB, 0, 0));
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      const int q = I + NB * i;
      Gr[r][i] = buf_load16(grs, (ok && q < NGL) ? (uint32_t)t * (uint32_t)gfb + q * 1024 + l * 16 : kOOB);
    }
    Cp[r] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                          crs, (ok && t >= 1) ? (uint32_t)(t - 1) * (uint32_t)bfb + bbase : kOOB, 0, 0));
    Mp[r] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                          mrs, ok ? (uint32_t)t * (uint32_t)sfb + sbase : kOOB, 0, 0));
    Bf[r] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                          brs, (!ERASE && ok) ? (uint32_t)t * (uint32_t)bfb + bbase : kOOB, 0, 0));
  };
  auto stage_g = [&](int slot, int r) {
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      const int q = I + NB * i;
      if (q < NGL) *(u32x4*)(gsl + (size_t)slot * Sh::g_slot + q * 1024 + l * 16) = Gr[r][i];
    }
  };
  auto g_half = [&](const unsigned char* gs, auto Lc) -> u32x2 {
    constexpr int L = decltype(Lc)::value;
    if constexpr (L >= NB) {
      return u32x2{0u, 0u};
    } else if constexpr (L <= I) {
      return *(const u32x2*)(gs + (size_t)(I * (I + 1) / 2 + L) * 512 + l * 8);
    } else {
      const unsigned char* blk = gs + (size_t)(L * (L + 1) / 2 + I) * 512;
      return lds_tr16((const uint16_t*)(blk + ((n & 3) * 16 + 4 * g + (n >> 2)) * 8));
    }
  };

#pragma unroll
  for (int r = 0; r < kStateRing; ++r) load_frame(r, r);
  stage_g(0, 0);
  lds_barrier();

  for (int base = 0; base < Tc; base += kStateRing) {
#pragma unroll
    for (int r = 0; r < kStateRing; ++r) {
      const int u = base + r, t = t_hi - 1 - u;
      const bool ok = u < Tc;
      const unsigned char* xr = xch + (size_t)(r & 1) * (Sh::xch_bytes / 2);
      const unsigned char* gs = gsl + (size_t)(r & 1) * Sh::g_slot;
      // bf16 snapshot of Lambda_t: the copy the waves exchanged
      __builtin_amdgcn_raw_buffer_store_b64(pub, lrs, ok ? (uint32_t)t * (uint32_t)sfb + sbase : kOOB, 0, 0);
      u32x4 aop[NKC], bop[NKC];
      static_for<NKC>([&](auto kbc) {
        constexpr int kb = decltype(kbc)::value;
        const u32x2 lo = g_half(gs, Int<2 * kb>{}), hi = g_half(gs, Int<2 * kb + 1>{});
        aop[kb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        bop[kb] = *(const u32x4*)(xr + ((size_t)kb * 64 + l) * 16);
      });
      __builtin_amdgcn_sched_barrier(0);
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) p = mfma_bf16(aop[kb], bop[kb], p);
      const float gm = Ga[r], bt = Be[r], bg = bt * gm;
      // partial sums over this wave's block
      const f32x4 mp = widen4(Mp[r]);
      float s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s1 += m[e] * mp[e];
        s2 += p[e] * mp[e];
      }
      if constexpr (!ERASE) {
        const f32x4 bw = widen4(Bf[r]);
#pragma unroll
        for (int e = 0; e < 4; ++e) s3 += m[e] * bw[e];
      }
#pragma unroll
      for (int sft = 32; sft >= 1; sft >>= 1) {
        s1 += __shfl_xor(s1, sft, 64);
        s2 += __shfl_xor(s2, sft, 64);
        if constexpr (!ERASE) s3 += __shfl_xor(s3, sft, 64);
      }
      const f32x4 ps = {s1, s2, s3, 0.f};
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, ps), prs,
          (ok && l == 0) ? (uint32_t)((t * NB * NB + j * NB + I) * 16) : kOOB, 0, 0);
      // Lambda_{t-1} = g Lambda_t - b g G_t Lambda_t + C_{t-1}
      const f32x4 cp = widen4(Cp[r]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float nv = gm * m[e] - bg * p[e] + cp[e];
        m[e] = ok ? nv : m[e];
      }
      stage_g((r + 1) & 1, (r + 1) % kStateRing);
      load_frame(u + kStateRing, r);
      pub = publish((r & 1) ^ 1, m);
      lds_barrier();
    }
  }
  if (a.lam_dst) {
    float* dst = a.lam_dst + (size_t)bh * D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(size_t)(row0 + r) * D + col] = m[r];
  }
}

template <int D, bool ERASE>
__global__ __launch_bounds__(D / 16 * 64, 1) void gdn_adjoint_bf16_kernel(AdjointArgs a) {
  constexpr int NB = D / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int unit = xcd_unit(a.BH * NB);
  if (unit < 0) return;
  const int bh = unit / NB, j = unit % NB;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  static_for<NB>([&](auto ic) {
    constexpr int I = decltype(ic)::value;
    if (w == I) adjoint_wave<D, ERASE, I>(a, smem, bh, j);
  });
}

// ----------------------------------------------------------------------------
// Launchers.
// ----------------------------------------------------------------------------
template <int D, bool FP8>
static hipError_t launch_gram_io(const GramArgs& ga, hipStream_t stream) {
  constexpr int NW = GramShape<D>::NW;
  static DeviceOnce once;
  LaunchInfo li;
  const hipError_t ie = once.get([](int dev, LaunchInfo& info) {
    hipError_t e = hipFuncSetAttribute((const void*)gdn_gram_kernel<D, FP8, NW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)GramShape<D>::lds_bytes);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)gdn_gram_kernel<D, FP8, 2 * NW, 2>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)(2 * GramShape<D>::lds_bytes));
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)gdn_gram_stream_kernel<D, FP8>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)GramStream<D>::lds_bytes);
    int per_cu = 0;
    if (e == hipSuccess) e = hipDeviceGetAttribute(&info.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)gdn_gram_stream_kernel<D, FP8>,
                                                       GramShape<D>::NW * 64, GramStream<D>::lds_bytes);
    info.slots = std::max(1, per_cu) * info.cus;
    return e;
  }, &li);
  if (ie != hipSuccess) return ie;
  const int cus = li.cus, slots = li.slots;
  const long long nfh = (long long)ga.BH * ga.Tc;
  const int nch = (ga.S + 31) / 32;
  if (ga.copy_src && nfh > 2 * cus) return hipErrorInvalidValue;   // only the short-launch kernels copy
  const unsigned grid = (unsigned)(nfh + (ga.copy_src ? ga.BH : 0));   // + one copy workgroup per head
  if (nfh <= 2 * cus) {
    // at most two frames per CU (a short streaming chunk): one workgroup per
    // frame with twice the waves, so that the launch takes half as long (four
    // times the waves measured slower again), and two chunks staged per
    // barrier (3 % faster than one)
    hipLaunchKernelGGL((gdn_gram_kernel<D, FP8, 2 * NW, 2>), dim3(grid), dim3(2 * NW * 64),
                       2 * GramShape<D>::lds_bytes, stream, ga);
  } else if (gram_stream_fits<D>() && nch >= gram_stream_min_chunks<D>()) {
    // persistent: one workgroup per resident slot
    const int grid = (int)std::min<long long>(nfh, slots);
    hipLaunchKernelGGL((gdn_gram_stream_kernel<D, FP8>), dim3(grid), dim3(GramShape<D>::NW * 64),
                       GramStream<D>::lds_bytes, stream, ga);
  } else {
    hipLaunchKernelGGL((gdn_gram_kernel<D, FP8, NW>), dim3((unsigned)nfh), dim3(NW * 64),
                       GramShape<D>::lds_bytes, stream, ga);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_gram_t(const GramArgs& ga, hipStream_t stream) {
  return ga.fp8 ? launch_gram_io<D, true>(ga, stream) : launch_gram_io<D, false>(ga, stream);
}

template <int D>
static hipError_t launch_state_t(const StateArgs& sa, hipStream_t stream) {
  static DeviceOnce once;
  LaunchInfo li;
  const hipError_t ie = once.get([](int, LaunchInfo&) {
    hipError_t e = hipFuncSetAttribute((const void*)gdn_state_bf16_kernel<D, true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)StateShape<D>::lds_bytes);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)gdn_state_bf16_kernel<D, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)StateShape<D>::lds_bytes);
    return e;
  }, &li);
  if (ie != hipSuccess) return ie;
  const int units = sa.BH * (D / 16);
  const int grid = 8 * ((units + 7) / 8);
  if (sa.beta_mode == 0)
    hipLaunchKernelGGL((gdn_state_bf16_kernel<D, true>), dim3(grid), dim3(D / 16 * 64), StateShape<D>::lds_bytes,
                       stream, sa);
  else
    hipLaunchKernelGGL((gdn_state_bf16_kernel<D, false>), dim3(grid), dim3(D / 16 * 64), StateShape<D>::lds_bytes,
                       stream, sa);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_step_tail_t(const TailArgs& ta, int cus, hipStream_t stream) {
  static DeviceOnce once;
  LaunchInfo li;
  const hipError_t ie = once.get([](int, LaunchInfo&) {
    const void* fns[4] = {(const void*)gdn_step_tail_kernel<D, false, true>,
                          (const void*)gdn_step_tail_kernel<D, false, false>,
                          (const void*)gdn_step_tail_kernel<D, true, true>,
                          (const void*)gdn_step_tail_kernel<D, true, false>};
    hipError_t e = hipSuccess;
    for (int i = 0; i < 4 && e == hipSuccess && tail_fits(D); ++i)
      e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)TailShape<D>::lds_bytes);
    return e;
  }, &li);
  if (ie != hipSuccess) return ie;
  if (!tail_fits(D) || ta.Tc < 1 || ta.Tc > kTailMaxFrames || ta.nsplit < 1) return hipErrorInvalidValue;
  const long long units = (long long)ta.BH * ta.Tc * ta.nsplit;
  if (units > (1ll << 30)) return hipErrorInvalidValue;
  (void)cus;
  const dim3 grid((unsigned)(8 * ((units + 7) / 8))), block(D / 16 * 64);
  const size_t lds = tail_fits(D) ? TailShape<D>::lds_bytes : 0;
  const bool erase = ta.beta_mode == 0;
  if (ta.fp8) {
    if (erase) hipLaunchKernelGGL((gdn_step_tail_kernel<D, true, true>), grid, block, lds, stream, ta);
    else hipLaunchKernelGGL((gdn_step_tail_kernel<D, true, false>), grid, block, lds, stream, ta);
  } else {
    if (erase) hipLaunchKernelGGL((gdn_step_tail_kernel<D, false, true>), grid, block, lds, stream, ta);
    else hipLaunchKernelGGL((gdn_step_tail_kernel<D, false, false>), grid, block, lds, stream, ta);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_cdq_t(const CdqArgs& ca, hipStream_t stream) {
  constexpr size_t lds = 5 * GramShape<D>::tile_bytes;   // Q, dO x 2 buffers; dQ tile
  static_assert((size_t)D * D * 2 <= 4 * GramShape<D>::tile_bytes, "snapshot staged in the tiles' space");
  static DeviceOnce once;
  LaunchInfo li;
  const hipError_t ie = once.get([](int, LaunchInfo&) {
    return hipFuncSetAttribute((const void*)gdn_cdq_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  }, &li);
  if (ie != hipSuccess) return ie;
  hipLaunchKernelGGL((gdn_cdq_kernel<D>), dim3((unsigned)(ca.BH * ca.Tc)), dim3(GramShape<D>::NW * 64), lds, stream,
                     ca);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_adjoint_t(const AdjointArgs& aa, hipStream_t stream) {
  static DeviceOnce once;
  LaunchInfo li;
  const hipError_t ie = once.get([](int, LaunchInfo&) {
    hipError_t e = hipFuncSetAttribute((const void*)gdn_adjoint_bf16_kernel<D, true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)StateShape<D>::lds_bytes);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)gdn_adjoint_bf16_kernel<D, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)StateShape<D>::lds_bytes);
    return e;
  }, &li);
  if (ie != hipSuccess) return ie;
  const int units = aa.BH * (D / 16);
  const int grid = 8 * ((units + 7) / 8);
  if (aa.beta_mode == 0)
    hipLaunchKernelGGL((gdn_adjoint_bf16_kernel<D, true>), dim3(grid), dim3(D / 16 * 64), StateShape<D>::lds_bytes,
                       stream, aa);
  else
    hipLaunchKernelGGL((gdn_adjoint_bf16_kernel<D, false>), dim3(grid), dim3(D / 16 * 64), StateShape<D>::lds_bytes,
                       stream, aa);
  return hipGetLastError();
}

#define GDN_DISPATCH(FN, ARGS)                                                 \
  switch (D) {                                                                 \
    case 16: return FN<16> ARGS;                                               \
    case 32: return FN<32> ARGS;                                               \
    case 48: return FN<48> ARGS;                                               \
    case 64: return FN<64> ARGS;                                               \
    case 80: return FN<80> ARGS;                                               \
    case 96: return FN<96> ARGS;                                               \
    case 112: return FN<112> ARGS;                                             \
    case 128: return FN<128> ARGS;                                             \
    default: return hipErrorInvalidValue;                                      \
  }

hipError_t launch_gram(int D, const GramArgs& ga, hipStream_t stream) {
  GDN_DISPATCH(launch_gram_t, (ga, stream))
}
hipError_t launch_state(int D, const StateArgs& sa, hipStream_t stream) {
  GDN_DISPATCH(launch_state_t, (sa, stream))
}
hipError_t launch_step_tail(int D, const TailArgs& ta, int cus, hipStream_t stream) {
  GDN_DISPATCH(launch_step_tail_t, (ta, cus, stream))
}
hipError_t launch_adjoint(int D, const AdjointArgs& aa, hipStream_t stream) {
  GDN_DISPATCH(launch_adjoint_t, (aa, stream))
}
hipError_t launch_cdq(int D, const CdqArgs& ca, hipStream_t stream) {
  GDN_DISPATCH(launch_cdq_t, (ca, stream))
}
#undef GDN_DISPATCH

size_t gram_frame_bytes(int D) {
  const size_t nb = (size_t)D / 16;
  return (nb * (nb + 1) / 2 + 1) / 2 * 1024;
}
size_t input_frame_bytes(int D) { return (size_t)(D / 16) * (D / 16) * 512; }

}  // namespace gdn
