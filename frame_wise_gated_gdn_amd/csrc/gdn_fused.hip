// Frame-wise Gated DeltaNet forward in one persistent launch (bf16 or e4m3
// I/O), on gfx950.
//
// The recurrence (SANA-WM news article "NVIDIA Apresenta SANA-WM ...",
// section "1. Atencao Linear Hibrida com Gated DeltaNet (GDN)") runs in the
// Gram form of gdn_gram.hip: per (head, frame) the frame-local terms
// G_t = Kf^T Kf and B_t = Kf^T V_t, the serial state update
// M_t = g M - b g G_t bf16(M) + B_t (B_t scaled by b in WRITE mode), and the
// readout O_t = ReLU(Q_t) bf16(M_t).  The three-pass pipeline moves G_t, B_t
// and the bf16 state copies through HBM between launches; here the three
// roles share one launch and hand those per-frame terms over through small
// rings that stay in the L2 of one XCD:
//
//   - head h's gram items and chain live on XCD h mod NX; two workgroups of
//     4 waves run on every CU (the launch's LDS request allows no third); the
//     chain workgroups of the XCD's heads sit in pairs on CUs of their own,
//     the rest are stream workgroups;
//   - with BH = q NX + rem, the readouts of the extra head of XCD x < rem run
//     on XCD x + rem, so that every XCD streams about the same bytes;
//   - a stream workgroup takes items of its XCD in a fixed order -- per
//     frame block u: the gram items G(h, u) of the XCD's heads, then the
//     readout items R(h, u - L) of its readout heads -- item k, k + Ns,
//     k + 2 Ns, ... for the k-th of Ns stream workgroups;
//   - G(h, t) reads K_t and V_t once (coalesced, non-temporal), and writes
//     G_t, B_t into slot t mod RG of the head's gram ring;
//   - the chain workgroups of h run the frames in order: G_t, B_t from the
//     ring, the state in fp32 registers (wave j of chain workgroup c owns
//     value tile 4c + j, every key block of it), the bf16 copy of M_t into
//     slot t mod RM of the head's state ring;
//   - R(h, t) reads the bf16 M_t from the ring and streams Q_t to O_t.
//
// Hand-over within an XCD: the producer's plain stores stay in that XCD's L2
// (write-back); it waits for them to complete, then stores a sequence number
// in a flag word.  The consumer polls the flag with device-scope loads, which
// miss the CU's L1 and read the L2, and then reads the data the same way.
// Gram items and chain of a head sit on the same XCD (each workgroup takes
// its role from its hardware XCC id), so there the L2 is the point of
// coherence and no L2 write-back or invalidation is needed.  The state copies
// and flags of a head whose readouts run on another XCD are written with
// device-scope stores, which write through the L2, and read there with
// device-scope loads.  Flags: per head, `cdone` (frames of the chain done:
// M_0..M_{cdone-1} are in the state ring, and the gram slots of those frames
// are free), `gready[s]` (1 + frame of the G_t, B_t in gram slot s) and
// `rdone[s]` (1 + frame whose state slot s has been read).
//
// Progress.  All workgroups are resident (cooperative launch).  The chain
// reads a frame's G three frames ahead and publishes `cdone` a frame late:
// in its step t it waits for the readout of frame t - RM (block t - RM + L)
// and the gram item of frame t + 3 (block t + 3), and cdone reaches t + 1 at
// the end of step t + 1.  So the readout R(h, t) (block t + L) waits on items
// of blocks up to t + 4 and t + 1 - RM + L, and the gram item G(h, u) (block
// u) on items of blocks up to u - RG + 4 and u - RG + 1 - RM + L.  Gram items
// precede the readouts of their block, so with 4 <= L, 5 <= RG and
// L <= RG + RM - 2 every wait is on an earlier item and the earliest
// unfinished item can always run.  Every wait is
// bounded: past kSpinLimit polls, or once another workgroup has given up,
// the workgroup sets the abort word (the first word of the control block)
// and leaves; the outputs of that launch are then incomplete.
//
// Arithmetic.  Each item repeats the three-pass kernels' operations in the
// same order (MFMA chains, scalings, roundings, the state update's fused
// multiply-adds, the norm's summation), so the results are bitwise those of
// the three-pass pipeline.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kFW = kFusedWaves;          // waves per workgroup
constexpr int kRingChunks = 2;            // gram item: 32-token chunks in flight per wave (even)
constexpr uint32_t kSpinLimit = 1u << 22; // polls before a wait gives up (far beyond any real wait)
constexpr int kCoherent = 16;             // cache bits of a device-scope load: miss L1, read L2
constexpr size_t kPairLds = 56 * 1024;    // LDS that keeps a CU at two workgroups

template <int D>
struct FShape {
  static constexpr int NB = D / 16;                   // 16-key (and 16-value) blocks
  static constexpr int NKC = (NB + 1) / 2;            // 32-key k-steps
  static constexpr int UPR = D / 8;                   // 16-byte units per token row (bf16)
  static constexpr int NLD = D / 16;                  // 1 KB pieces per 32-token chunk of one tensor
  static constexpr int RS = D + 8;                    // LDS row stride (elements)
  static constexpr int RS8 = D + 8;                   // row stride of an e4m3 tile (bytes; rows 8 bytes
                                                      // off a 16-byte grid keep the transposing reads apart)
  static constexpr size_t tile_bytes = (size_t)32 * RS * 2;
  static constexpr int NBLK = NB * (NB + 1) / 2;      // stored G blocks (I >= L)
  static constexpr int NBB = NB * NB;                 // B blocks
  static constexpr int NOUT = NBB + NBLK;
  static constexpr size_t g_bytes = (size_t)(NBLK + 1) / 2 * 1024;   // G part of a gram slot
  static constexpr size_t b_bytes = (size_t)NBB * 512;               // B part
  static constexpr size_t slot_bytes = g_bytes + b_bytes;
  static constexpr int NGL = (int)(g_bytes / 1024);   // 1 KB pieces of G
  static constexpr size_t gram_lds = 4 * tile_bytes;  // (K, V) x 2 buffers
  static constexpr size_t read_lds = (size_t)kFW * tile_bytes;       // per wave a Q (then O) tile
  static constexpr size_t read_all = read_lds + (size_t)D * D * 2;  // + M_t
  static constexpr size_t chain_lds = 3 * g_bytes;    // three G slots
  static constexpr size_t lds_bytes = (gram_lds > read_all ? (gram_lds > chain_lds ? gram_lds : chain_lds)
                                                           : (read_all > chain_lds ? read_all : chain_lds)) +
                                      64;             // + broadcast words
  // requested at launch: at least a third of the CU's 160 KB, so that a CU
  // holds two workgroups and never three
  static constexpr size_t launch_lds = lds_bytes > kPairLds ? lds_bytes : kPairLds;
};

// stored G block k = I(I+1)/2 + L (I >= L) -> I, L
constexpr int fblk_row(int k) {
  int I = 0;
  while ((I + 1) * (I + 2) / 2 <= k) ++I;
  return I;
}
constexpr int fblk_col(int k) { return k - fblk_row(k) * (fblk_row(k) + 1) / 2; }
constexpr uint32_t fxmask(int NB, int b0, int b1) {
  uint32_t m = 0;
  for (int b = b0; b < b1; ++b) {
    if (b < NB * NB) {
      m |= 1u << (b % NB);
    } else {
      m |= 1u << fblk_row(b - NB * NB);
      m |= 1u << fblk_col(b - NB * NB);
    }
  }
  return m;
}
constexpr uint32_t fymask(int NB, int b0, int b1) {
  uint32_t m = 0;
  for (int b = b0; b < b1 && b < NB * NB; ++b) m |= 1u << (b / NB);
  return m;
}

// ---------------------------------------------------------------------------
// Flags and waits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t* head_ctl(const FusedArgs& a, int h) {
  return (uint32_t*)(a.ctl + kFusedCtlHead + (size_t)h * kFusedCtlPerHead);
}
// chain workgroups per head: one per 4 value tiles (one tile per wave)
template <int D>
constexpr int chain_wgs() { return (D / 16 + kFusedWaves - 1) / kFusedWaves; }
__device__ __forceinline__ uint32_t* cdone_flag(const FusedArgs& a, int h, int c) { return head_ctl(a, h) + 16 * c; }
__device__ __forceinline__ uint32_t* gready_flag(const FusedArgs& a, int h, int s) {
  return head_ctl(a, h) + 16 * (kFusedMaxCW + s);
}
__device__ __forceinline__ uint32_t* rdone_flag(const FusedArgs& a, int h, int s) {
  return head_ctl(a, h) + 16 * (kFusedMaxCW + kFusedMaxRG + s);
}
__device__ __forceinline__ uint32_t poll(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // device scope: L1 miss
}
__device__ __forceinline__ void flag_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);  // a plain store: stays in L2
}
// A flag read on other XCDs: a device-scope store, written through the L2
__device__ __forceinline__ void flag_store_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until *p >= target, polled by the calling wave (all lanes see the
// same values).  Returns false when the wait gave up (abort word set here or
// by another workgroup).
__device__ __forceinline__ bool wait_geq(const FusedArgs& a, const uint32_t* p, uint32_t target) {
  uint32_t* abort_word = (uint32_t*)a.ctl;
  for (uint32_t n = 0;; ++n) {
    const uint32_t v = __builtin_amdgcn_readfirstlane(poll(p));
    if (v >= target) return true;
    if ((n & 31) == 31 && __builtin_amdgcn_readfirstlane(poll(abort_word)) != 0) return false;
    if (n >= kSpinLimit) {
      flag_store_dev(abort_word, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}
// Wait until every chain workgroup of head h has published at least `target`.
template <int CW>
__device__ __forceinline__ bool wait_chain(const FusedArgs& a, int h, uint32_t target) {
  bool ok = true;
#pragma unroll
  for (int c = 0; c < CW; ++c) ok = ok && wait_geq(a, cdone_flag(a, h, c), target);
  return ok;
}
template <int CW>
__device__ __forceinline__ uint32_t poll_chain(const FusedArgs& a, int h) {
  uint32_t v = 0xffffffffu;
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    const uint32_t x = __builtin_amdgcn_readfirstlane(poll(cdone_flag(a, h, c)));
    v = x < v ? x : v;
  }
  return v;
}
// Waits for this wave's outstanding memory operations (stores included).
__device__ __forceinline__ void wait_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier that also hands wave 0's verdict to every wave, with one
// s_barrier per call: the word written alternates between two, and a word is
// written again only two calls later, once every wave has passed the barrier
// in between (and so has read it).  Every wave makes the same calls.
struct Bcast {
  uint32_t* w;     // two words in LDS
  uint32_t n;
  __device__ __forceinline__ bool sync(bool ok_wave0) {
    uint32_t* p = w + (n & 1u);
    ++n;
    if ((threadIdx.x >> 6) == 0 && lane_id() == 0) *p = ok_wave0 ? 1u : 0u;
    __syncthreads();
    return *(volatile uint32_t*)p != 0;
  }
};

__device__ __forceinline__ unsigned char* gslot(const FusedArgs& a, int h, int s, size_t slot_bytes) {
  return a.gring + ((size_t)h * a.RG + s) * slot_bytes;
}
__device__ __forceinline__ unsigned char* mslot(const FusedArgs& a, int h, int s, int D) {
  return a.mring + ((size_t)h * a.RM + s) * (size_t)D * D * 2;
}

// ---------------------------------------------------------------------------
// Gram item G(h, t): wave W of 4 owns output blocks [W NOUT/4, (W+1) NOUT/4)
// of (B blocks, then stored G blocks), exactly as the gram kernels split
// them among their waves; every block is accumulated over the 32-token
// chunks in order, one MFMA per chunk.
// ---------------------------------------------------------------------------
template <int D, bool FP8, int W>
__device__ __forceinline__ bool gram_item_wave(const FusedArgs& a, unsigned char* smem, Bcast& bc, int h,
                                               int t) {
  using Sh = FShape<D>;
  using IO = IoFmt<FP8>;
  using raw = typename IO::raw;
  constexpr int NB = Sh::NB, UPR = Sh::UPR, NLD = Sh::NLD, RS = Sh::RS, NW = kFW;
  constexpr int LPW = (2 * NLD + NW - 1) / NW;
  constexpr int NBB = Sh::NBB, NOUT = Sh::NOUT;
  constexpr int B0 = W * NOUT / NW, B1 = (W + 1) * NOUT / NW, NMB = B1 - B0;
  constexpr uint32_t XM = fxmask(NB, B0, B1), YM = fymask(NB, B0, B1);
  const int l = lane_id(), g = l >> 4, n = l & 15;
  const int S = a.S, T = a.T;
  const uint32_t frame_bytes = (uint32_t)S * D * IO::ebytes;
  const size_t fe = ((size_t)h * T + t) * frame_bytes;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc((const unsigned char*)a.k + fe, frame_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const unsigned char*)a.v + fe, frame_bytes);
  const int nch = (S + 31) / 32;
  const int nit = (nch + kRingChunks - 1) / kRingChunks * kRingChunks;

  auto load_chunk = [&](int ch, raw (&X)[LPW]) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int p = W + NW * i;
      const int u = 64 * (p % NLD) + l;
      const int tok = ch * 32 + u / UPR;
      const bool ok = p < 2 * NLD && ch < nch && tok < S;
      const uint32_t off = ok ? (uint32_t)(ch * 32 * UPR + u) * IO::unit_bytes : kOOB;
      X[i] = IO::load_nt(p < NLD ? krs : vrs, off);
    }
  };
  // bf16 I/O: the chunk is staged as bf16 (K through ReLU) and the blocks
  // are bf16 MFMAs; e4m3 I/O: staged as e4m3 codes, fp8 MFMAs (exact
  // products, sums within about 2^-12 of the sum of |products|), the gram
  // kernel's e4m3 form, so both give the same bits
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
  // e4m3 operand of block blk: dim 16 blk + l % 16, tokens 8 (l / 16) .. + 7
  auto frag8 = [&](const unsigned char* tile, int blk) -> u32x2 {
    return lds_tr8(tile + (8 * g + (n >> 1)) * Sh::RS8 + 16 * blk + 8 * (n & 1));
  };

  f32x4 acc[NMB > 0 ? NMB : 1];
#pragma unroll
  for (int i = 0; i < NMB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the ring slot of frame t must have been consumed (frame t - RG done):
  // polled now, checked before the stores
  constexpr int CW = chain_wgs<D>();
  const uint32_t pslot = (W == 0 && t >= a.RG) ? poll_chain<CW>(a, h) : 0u;
  raw R[kRingChunks][LPW];
#pragma unroll
  for (int r = 0; r < kRingChunks; ++r) load_chunk(r, R[r]);
  for (int base = 0; base < nit; base += kRingChunks) {
#pragma unroll
    for (int r = 0; r < kRingChunks; ++r) {
      const int c = base + r;
      stage(r & 1, R[r]);
      load_chunk(c + kRingChunks, R[r]);
      lds_barrier();
      if (c < nch && FP8) {
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
            acc[i] = mfma_fp8(X[fblk_col(k)], X[fblk_row(k)], acc[i]);
          }
        });
      } else if (c < nch) {
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
            acc[i] = mfma_bf16(X[fblk_col(k)], X[fblk_row(k)], acc[i]);
          }
        });
      }
    }
  }

  const int s = t % a.RG;
  bool ok = true;
  if (W == 0 && t >= a.RG && pslot < (uint32_t)(t - a.RG + 1)) ok = wait_chain<CW>(a, h, (uint32_t)(t - a.RG + 1));
  if (!bc.sync(ok)) return false;
  unsigned char* gout = gslot(a, h, s, Sh::slot_bytes);
  unsigned char* bout = gout + Sh::g_bytes;
  const float c2 = a.kscale2, c1 = a.kscale;
  static_for<NMB>([&](auto ic) {
    constexpr int i = decltype(ic)::value, b = B0 + i;
    const f32x4 x = acc[i];
    if constexpr (b < NBB) {
      const u32x2 v = {pack_bf16(c1 * x[0], c1 * x[1]), pack_bf16(c1 * x[2], c1 * x[3])};
      *(u32x2*)(bout + (size_t)b * 512 + l * 8) = v;
    } else {
      const u32x2 v = {pack_bf16(c2 * x[0], c2 * x[1]), pack_bf16(c2 * x[2], c2 * x[3])};
      *(u32x2*)(gout + (size_t)(b - NBB) * 512 + l * 8) = v;
    }
  });
  wait_memory();
  __syncthreads();
  if (W == 0 && l == 0) flag_store(gready_flag(a, h, s), (uint32_t)(t + 1));
  return true;
}

// ---------------------------------------------------------------------------
// Readout item R(h, t): the 4 waves split the frame's 32-token chunks as the
// readout kernel does.  M_t comes from the state ring into LDS (block
// layout), and every wave reads its A operands (M_t^T rows) from there once
// per chunk for both 16-token halves; the O chunk is assembled in place of
// the staged ReLU(Q) chunk, whose B operands are then all in registers.  Per
// output element the MFMA chain over the k-steps is the readout kernel's.
// ---------------------------------------------------------------------------
template <int D, bool FP8>
__device__ __forceinline__ bool readout_item(const FusedArgs& a, unsigned char* smem, Bcast& bc, int h,
                                             int t, bool remote) {
  using Sh = FShape<D>;
  using IO = IoFmt<FP8>;
  using raw = typename IO::raw;
  constexpr int NB = Sh::NB, NKC = Sh::NKC, UPR = Sh::UPR, NLD = Sh::NLD, RS = Sh::RS, RW = kFW;
  constexpr int RS8 = D + 8;
  constexpr int CW = chain_wgs<D>();
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, n = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint16_t* const qs = (uint16_t*)(smem + (size_t)w * Sh::tile_bytes);   // ReLU(Q) chunk, then O chunk
  unsigned char* const msm = smem + Sh::read_lds;                         // M_t (bf16, block layout)
  const int S = a.S, T = a.T;
  const uint32_t head_bytes = (uint32_t)T * (uint32_t)S * D * IO::ebytes;
  const size_t head0 = (size_t)h * T * S * D * IO::ebytes;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc((const unsigned char*)a.q + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t ors = make_rsrc((unsigned char*)a.o + head0, head_bytes);
  const uint32_t fbyte = (uint32_t)t * (uint32_t)S * D * IO::ebytes;
  const int nchunk = (S + 31) / 32;
  const int NC = (nchunk + RW - 1) / RW;

  auto unit_off = [&](int ch, int u) -> uint32_t {
    const int tok = ch * 32 + u / UPR;
    return (ch < nchunk && tok < S) ? fbyte + (uint32_t)(ch * 32 * UPR + u) * IO::unit_bytes : kOOB;
  };
  auto load_chunk = [&](int i, raw (&X)[NLD]) {
    const int ch = w + RW * i;
#pragma unroll
    for (int j = 0; j < NLD; ++j) X[j] = IO::load_nt(qrs, i < NC ? unit_off(ch, 64 * j + l) : kOOB);
  };
  // M_t must be in the state ring: polled now, checked once the first Q
  // chunks are on their way
  const uint32_t pc = w == 0 ? poll_chain<CW>(a, h) : 0u;
  constexpr int RING = 3;                                             // Q chunks in flight per wave
  raw X[RING][NLD];
#pragma unroll
  for (int r = 0; r < RING; ++r) load_chunk(r, X[r]);
  bool ok = true;
  if (w == 0 && pc < (uint32_t)(t + 1)) ok = wait_chain<CW>(a, h, (uint32_t)(t + 1));
  if (!bc.sync(ok)) return false;
  const int s = t % a.RM;
  {
    constexpr int NU = D * D * 2 / 16;                                    // 16-byte units of M_t
    const __amdgpu_buffer_rsrc_t mrs = make_rsrc(mslot(a, h, s, D), (uint32_t)(D * D * 2));
    for (int u = tid; u < NU; u += RW * 64) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(mrs, (uint32_t)u * 16u, 0,
                                                                                        kCoherent));
      *(u32x4*)(msm + (size_t)u * 16) = v;
    }
  }
  __syncthreads();                                   // M_t in LDS: the loads are done, the slot may be refilled
  if (w == 0 && l == 0) {
    if (remote) flag_store_dev(rdone_flag(a, h, s), (uint32_t)(t + 1));
    else flag_store(rdone_flag(a, h, s), (uint32_t)(t + 1));
  }
  // A operand (jb, kc) of this lane: blocks (jb, 2kc) and (jb, 2kc + 1)
  auto a_frag = [&](int jb, int kc) -> u32x4 {
    const u32x2 lo = *(const u32x2*)(msm + ((size_t)(jb * NB + 2 * kc) * 64 + l) * 8);
    const u32x2 hi = (2 * kc + 1 < NB) ? *(const u32x2*)(msm + ((size_t)(jb * NB + 2 * kc + 1) * 64 + l) * 8)
                                       : u32x2{0u, 0u};
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  if (a.norms && w == 0) {
    // state norm from the bf16 copy, summed as the readout kernel sums it
    float sq = 0.f;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const u32x4 af = a_frag(jb, kc);
#pragma unroll
        for (int e = 0; e < 4; ++e) sq = add_sq_bf16x2(sq, af[e]);
      }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) sq += __shfl_xor(sq, sh, 64);
    if (l == 0) a.norms[(size_t)h * T + t] = sqrtf(sq);
  }

  for (int base = 0; base < NC; base += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int i = base + r;
      const int ch = w + RW * i;
      const bool live = i < NC;
      if (live) {
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
          const int u = 64 * j + l;
          *(u32x4*)(qs + (u / UPR) * RS + 8 * (u % UPR)) = relu8(IO::to_bf16(X[r][j]));
        }
      }
      load_chunk(i + RING, X[r]);
      if (!live) continue;
      wave_lds_sync();
      u32x4 Bq[2][NKC];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          const uint16_t* rp = qs + (16 * half + n) * RS + 32 * kc + 4 * g;
          const u32x2 lo = *(const u32x2*)rp;
          const u32x2 hi = (32 * kc + 32 <= D) ? *(const u32x2*)(rp + 16) : u32x2{0u, 0u};
          Bq[half][kc] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      wave_lds_sync();                                                     // the chunk is in registers
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        u32x4 Af[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) Af[kc] = a_frag(jb, kc);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) acc = mfma_bf16(Af[kc], Bq[half][kc], acc);
          if constexpr (FP8) {
            *(uint32_t*)((unsigned char*)qs + (16 * half + n) * RS8 + 16 * jb + 4 * g) = f32x4_to_fp8x4(acc);
          } else {
            const u32x2 pk = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
            *(u32x2*)(qs + (16 * half + n) * RS + 16 * jb + 4 * g) = pk;
          }
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int u = 64 * j + l;
        if constexpr (FP8) {
          const u32x2 y = *(const u32x2*)((const unsigned char*)qs + (u / UPR) * RS8 + 8 * (u % UPR));
          __builtin_amdgcn_raw_buffer_store_b64(y, ors, unit_off(ch, u), 0, kNT);
        } else {
          const u32x4 y = *(const u32x4*)(qs + (u / UPR) * RS + 8 * (u % UPR));
          __builtin_amdgcn_raw_buffer_store_b128(y, ors, unit_off(ch, u), 0, kNT);
        }
      }
    }
  }
  return true;
}

// ---------------------------------------------------------------------------
// Chain workgroup c of head h: wave J owns value tile j = 4c + J (all NB key
// blocks of it) in fp32; per frame it forms (G_t bf16(M_{t-1}))[I][j] for
// every key block I with NKC MFMAs each -- A operands from the frame's stored
// G blocks in LDS, the B operand from the wave's own registers (its
// accumulator layout is the k-slot order of the operand) -- then the gate,
// the input term and the erase, exactly as the state pass does for block
// (I, j).  Value tiles evolve independently, so the chain workgroups of a
// head only share their inputs.
// ---------------------------------------------------------------------------
// J is a run-time value on purpose: the four waves then run one copy of the
// frame loop, which stays in the instruction cache.
template <int D, bool ERASE, bool REMOTE>
__device__ __forceinline__ void chain_wave(const FusedArgs& a, unsigned char* smem, int h, int c, const int J) {
  using Sh = FShape<D>;
  constexpr int NB = Sh::NB, NKC = Sh::NKC, NGL = Sh::NGL;
  constexpr int LPG = (NGL + kFW - 1) / kFW;         // G pieces loaded per wave
  const int l = lane_id(), g = l >> 4, n = l & 15;
  const int T = a.T;
  const int j = kFW * c + J;                         // value tile of this wave
  const bool own = j < NB;                           // waves past NB only help with G
  unsigned char* const gsl = smem;                   // three G slots

  f32x4 m[NB];
  const int col = 16 * (own ? j : 0) + n;
#pragma unroll
  for (int I = 0; I < NB; ++I) {
    m[I] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (own && a.state_in) {
      const float* src = a.state_in + (size_t)h * D * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) m[I][r] = src[(size_t)(16 * I + 4 * g + r) * D + col];
    }
  }
  const __amdgpu_buffer_rsrc_t gars = make_rsrc(a.gamma + (size_t)h * T, (uint32_t)(T * 4));
  const __amdgpu_buffer_rsrc_t bers = make_rsrc(a.beta + (size_t)h * T, (uint32_t)(T * 4));
  auto slot_rsrc = [&](int f) {
    return make_rsrc(gslot(a, h, f < T ? f % a.RG : 0, Sh::slot_bytes), (uint32_t)Sh::slot_bytes);
  };

  // Register buffers (the frame loop is unrolled by two, so every buffer
  // index is a constant): Gr[f & 1] holds this wave's G pieces of frame f from
  // their load (during frame f - 3) to their staging (during frame f - 2);
  // Bn[f & 1], ga[f & 1], be[f & 1] frame f's B blocks, gamma and beta from
  // their load (during frame f - 2, after frame f - 2's update has read the
  // buffer) to their use: two frames of memory latency, which a saturated
  // HBM needs.
  u32x4 Gr[2][LPG];
  u32x2 Bn[2][NB];
  float ga[2] = {0.f, 0.f}, be[2] = {0.f, 0.f};
  auto load_g = [&](int f, auto bc_) {
    constexpr int r = decltype(bc_)::value;
    const bool ok = f < T;
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc(f);
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      const int q = J + kFW * i;
      Gr[r][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rs, (ok && q < NGL) ? (uint32_t)(q * 1024 + l * 16) : kOOB, 0,
                                               kCoherent));
    }
  };
  auto load_b = [&](int f, auto bc_) {
    constexpr int r = decltype(bc_)::value;
    const bool ok = f < T;                           // issued in any case (out of range: no access)
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc(f);
    ga[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gars, ok ? (uint32_t)f * 4u : kOOB, 0, 0));
    be[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(bers, ok ? (uint32_t)f * 4u : kOOB, 0, 0));
#pragma unroll
    for (int I = 0; I < NB; ++I)
      Bn[r][I] = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                     rs, (ok && own) ? (uint32_t)(Sh::g_bytes + ((j * NB + I) * 512 + l * 8)) : kOOB, 0, kCoherent));
  };
  auto stage_g = [&](int f, auto bc_) {             // buffer r's G (frame f) into LDS slot f mod 3
    constexpr int r = decltype(bc_)::value;
    unsigned char* dst = gsl + (size_t)(f % 3) * Sh::g_bytes;
    asm volatile("" ::"v"(Gr[r][LPG - 1]));
#pragma unroll
    for (int i = 0; i < LPG; ++i) {
      const int q = J + kFW * i;
      if (q < NGL) *(u32x4*)(dst + q * 1024 + l * 16) = Gr[r][i];
    }
  };
  // A operand half for key block I, k-block L: row n of block (I, L), columns 4g..4g+3
  auto g_half = [&](const unsigned char* gs, auto Ic, auto Lc) -> u32x2 {
    constexpr int I = decltype(Ic)::value, L = decltype(Lc)::value;
    if constexpr (L >= NB) {
      return u32x2{0u, 0u};
    } else if constexpr (L <= I) {
      return *(const u32x2*)(gs + (size_t)(I * (I + 1) / 2 + L) * 512 + l * 8);
    } else {
      const unsigned char* blk = gs + (size_t)(L * (L + 1) / 2 + I) * 512;
      return lds_tr16((const uint16_t*)(blk + ((n & 3) * 16 + 4 * g + (n >> 2)) * 8));
    }
  };

  // Frame f, per wave: the MFMAs and the update (G from LDS slot f mod 3, B
  // and the gates from registers); the check that frame f - RM's readout has
  // copied its state slot; the polls for frame f + 1; frame f + 2's B and
  // gates into registers; the bf16 M_f into the state ring; the check that
  // gram slot f + 3 is filled and its G into registers; frame f + 2's G
  // (loaded during frame f - 1) into LDS slot (f + 2) mod 3; then the one
  // barrier of the frame, after which cdone = f.  Each wave checks the flags
  // its own loads and stores depend on, so no barrier waits on a broadcast.
  // A wave's vector memory operations complete in order: once every wave has
  // its frame f + 2 G back, the M_{f-1} stores issued before those loads are
  // in the L2 (cdone = f: M_0..M_{f-1} stored), and the loads of frames up to
  // f are complete (their gram slots are free).  The same memory operations
  // are issued on every path (out-of-range offsets where there is nothing to
  // do), so the waits the compiler places for a value cover exactly the
  // operations issued up to that value's load: each wait is on loads issued
  // at least a frame earlier.  A wave whose wait gave up (abort word set)
  // stops waiting and runs to the end, so the barriers still match.
  auto gready_of = [&](int f) { return gready_flag(a, h, f % a.RG); };
  auto rdone_of = [&](int f) { return rdone_flag(a, h, f % a.RM); };
  uint32_t* const cdone = cdone_flag(a, h, c);
  bool live = true;
  auto check = [&](uint32_t polled, const uint32_t* flag, uint32_t target) {
    if (live && __builtin_amdgcn_readfirstlane(polled) < target) live = wait_geq(a, flag, target);
  };
  auto store_flag = [&](uint32_t v) {
    if constexpr (REMOTE) flag_store_dev(cdone, v);
    else flag_store(cdone, v);
  };
  const __amdgpu_buffer_rsrc_t mring_rs = make_rsrc(mslot(a, h, 0, D), (uint32_t)(a.RM * D * D * 2));
  for (int f = 0; f < 3 && f < T; ++f) check(0u, gready_of(f), (uint32_t)(f + 1));
  load_g(0, Int<0>{});
  load_g(1, Int<1>{});
  stage_g(0, Int<0>{});
  stage_g(1, Int<1>{});
  uint32_t pr[2], pg[2];              // polled rdone of frame f's state slot, gready of frame f + 3
  // the state stores of a frame (none here: out of range); the prologue
  // issues what a frame issues, in the same order, so that the loop entry
  // and the loop back edge agree on the operations in flight
  auto store_m = [&](int f) {
    const uint32_t base = (uint32_t)((f % a.RM) * D * D * 2);
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      const u32x2 pub = {pack_bf16(m[I][0], m[I][1]), pack_bf16(m[I][2], m[I][3])};
      const uint32_t off = (own && f >= 0) ? base + (uint32_t)(((j * NB + I) * 64 + l) * 8) : kOOB;
      // a state read on another XCD is written through the L2
      __builtin_amdgcn_raw_buffer_store_b64(pub, mring_rs, off, 0, REMOTE ? kCoherent : 0);
    }
  };
  load_b(0, Int<0>{});
  pr[0] = poll(rdone_of(0));
  pg[0] = poll(gready_of(3));
  load_b(1, Int<1>{});
  store_m(-1);
  load_g(2, Int<0>{});
  __syncthreads();

  auto frame = [&](auto rc, int f) {
    constexpr int r = decltype(rc)::value;
    if (own) {
      const unsigned char* gs = gsl + (size_t)(f % 3) * Sh::g_bytes;
      const float gm = ga[r], bt = be[r], bg = bt * gm;
      // B operand: bf16 of the state column tile in k-slot order
      u32x4 bop[NKC];
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) {
        const f32x4 lo = m[2 * kb];
        const u32x2 plo = {pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3])};
        u32x2 phi = {0u, 0u};
        if (2 * kb + 1 < NB) {
          const f32x4 hi = m[2 * kb + 1];
          phi = u32x2{pack_bf16(hi[0], hi[1]), pack_bf16(hi[2], hi[3])};
        }
        bop[kb] = u32x4{plo[0], plo[1], phi[0], phi[1]};
      }
      static_for<NB>([&](auto Ic) {
        constexpr int I = decltype(Ic)::value;
        u32x4 aop[NKC];
        static_for<NKC>([&](auto kbc) {
          constexpr int kb = decltype(kbc)::value;
          const u32x2 lo = g_half(gs, Ic, Int<2 * kb>{}), hi = g_half(gs, Ic, Int<2 * kb + 1>{});
          aop[kb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        });
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) acc = mfma_bf16(aop[kb], bop[kb], acc);
        const u32x2 bw = Bn[r][I];
        const f32x4 bin = {bf16_lo_f32(bw[0]), bf16_hi_f32(bw[0]), bf16_lo_f32(bw[1]), bf16_hi_f32(bw[1])};
#pragma unroll
        for (int e = 0; e < 4; ++e) m[I][e] = state_update(gm, m[I][e], bg, acc[e], ERASE ? bin[e] : bt * bin[e]);
      });
      // the state slot of frame f must have been read (frame f - RM done)
      if (f >= a.RM) check(pr[r], rdone_of(f), (uint32_t)(f - a.RM + 1));
    }
    pr[r ^ 1] = poll(rdone_of(f + 1));
    pg[r ^ 1] = poll(gready_of(f + 4));
    load_b(f + 2, Int<r>{});
    store_m(f);
    if (f + 3 < T) check(pg[r], gready_of(f + 3), (uint32_t)(f + 4));
    load_g(f + 3, Int<r ^ 1>{});
    stage_g(f + 2, Int<r>{});
    __syncthreads();
    if (J == 0 && l == 0 && f >= 1 && live) store_flag((uint32_t)f);
  };
  int t = 0;
  for (; t + 1 < T; t += 2) {
    frame(Int<0>{}, t);
    frame(Int<1>{}, t + 1);
  }
  if (t < T) frame(Int<0>{}, t);
  wait_memory();
  __syncthreads();
  if (J == 0 && l == 0 && live) store_flag((uint32_t)T);
  if (own && a.state_out) {
    float* dst = a.state_out + (size_t)h * D * D;
#pragma unroll
    for (int I = 0; I < NB; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(16 * I + 4 * g + r) * D + col] = m[I][r];
  }
}

template <int D, bool FP8, bool ERASE>
__global__ __launch_bounds__(kFusedWaves * 64, 2) void gdn_fused_kernel(FusedArgs a) {
  using Sh = FShape<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Bcast bc{(uint32_t*)(smem + Sh::lds_bytes - 64), 0u};
  uint32_t* bcast = bc.w + 2;                                          // the ticket's broadcast word
  const int NX = a.NX;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The XCD this workgroup runs on and its CU, from the hardware.  The
  // dispatcher deals workgroups to the XCDs round-robin, grid/NX to each, but
  // the XCD of workgroup 0 depends on earlier launches, so the workgroup id
  // does not tell; and every CU holds exactly two workgroups (the launch
  // size and its LDS request).  The first of a CU's two takes the CU's rank
  // among the CUs of its XCD (a ticket) and posts it; the second reads it.
  // p = 2 rank + (0 or 1) numbers the XCD's workgroups so that p and p ^ 1
  // share a CU: the chain workgroups, p < nh CW, then sit in pairs on CUs of
  // their own, away from the streaming workgroups' memory traffic.
  uint32_t xcc, hwid;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hwid));
  const int x = (int)(xcc & 0xFu);
  const int nwg = (int)gridDim.x / NX;                                 // workgroups on each XCD
  if (threadIdx.x == 0) {
    uint32_t pos = 0xffffffffu;
    if (x < NX) {
      uint32_t* cu = (uint32_t*)(a.ctl + kFusedCtlCu + ((size_t)x * 256 + ((hwid >> 8) & 0xFFu)) * 8);
      const uint32_t slot = __hip_atomic_fetch_add(cu, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (slot == 0) {
        const uint32_t rank = __hip_atomic_fetch_add((uint32_t*)(a.ctl + kFusedCtlTicket + 64 * x), 1u,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        flag_store(cu + 1, rank + 1u);
        pos = 2 * rank;
      } else if (slot == 1 && wait_geq(a, cu + 1, 1u)) {
        pos = 2 * (poll(cu + 1) - 1u) + 1u;
      }
    }
    *bcast = pos;
  }
  __syncthreads();
  const int rank = (int)__builtin_amdgcn_readfirstlane(*(volatile uint32_t*)bcast);
  __syncthreads();
  if (x >= NX || rank < 0 || rank >= nwg) {
    // an XCD with more workgroups than its share, or a CU with more than two
    if (threadIdx.x == 0) flag_store_dev((uint32_t*)a.ctl, 2u);
    return;
  }
  constexpr int CW = chain_wgs<D>();
  // Heads: head h's gram items and chain on XCD h mod NX.  With BH = q NX +
  // rem and a.balance set, the XCDs x < rem hold one head more than the
  // others; the readouts of that last head go to XCD x + rem (when it
  // exists), so that every XCD then streams about the same bytes.  Such a
  // head's state copies and flags are written through the L2 (device-scope
  // stores), read with device-scope loads on the other XCD.
  const int q = a.BH / NX, rem = a.BH % NX;
  const int nh = x < a.BH ? (a.BH - x + NX - 1) / NX : 0;              // heads of this XCD
  const bool moved = a.balance && x < rem && x + rem < NX;             // last head's readouts elsewhere
  const bool incoming = a.balance && x >= rem && x < 2 * rem;          // readouts of head x - rem + q NX here
  const int nr = nh - (moved ? 1 : 0) + (incoming ? 1 : 0);            // readout heads
  if (rank < nh * CW) {
    const int hi = rank / CW, h = x + NX * hi, c = rank % CW;
    const bool remote = moved && hi == nh - 1;
    if (remote) chain_wave<D, ERASE, true>(a, smem, h, c, w);
    else chain_wave<D, ERASE, false>(a, smem, h, c, w);
    return;
  }
  const int ns = nwg - nh * CW, k = rank - nh * CW;                    // stream workgroups of this XCD
  if (nh + nr == 0) return;
  if (ns <= 0) {
    if (threadIdx.x == 0) flag_store_dev((uint32_t*)a.ctl, 3u);         // no stream workgroup: give up
    return;
  }
  const long long per_block = (long long)nh + nr;
  const long long nitems = per_block * (long long)(a.T + a.L);
  for (long long it = k; it < nitems; it += ns) {
    const int u = (int)(it / per_block), r = (int)(it % per_block);
    bool ok = true;
    if (r < nh) {
      if (u >= a.T) continue;
      const int h = x + NX * r;
      static_for<kFW>([&](auto wc) {
        constexpr int W = decltype(wc)::value;
        if (w == W) ok = gram_item_wave<D, FP8, W>(a, smem, bc, h, u);
      });
    } else {
      const int t = u - a.L;
      if (t < 0 || t >= a.T) continue;
      const int ri = r - nh;
      const bool remote = incoming && ri == nr - 1;
      ok = readout_item<D, FP8>(a, smem, bc, remote ? x - rem + NX * q : x + NX * ri, t, remote);
    }
    if (!ok) return;
    __syncthreads();                                                   // LDS reuse by the next item
  }
}

__global__ void gdn_fused_clear_kernel(uint32_t* p, uint32_t words) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < words; i += gridDim.x * blockDim.x) p[i] = 0u;
}

template <int D, bool FP8, bool ERASE>
hipError_t launch_fused_t3(const FusedArgs& fa, int grid, hipStream_t stream) {
  const void* fn = (const void*)gdn_fused_kernel<D, FP8, ERASE>;
  FusedArgs arg = fa;
  void* params[] = {&arg};
  return hipLaunchCooperativeKernel(fn, dim3((unsigned)grid), dim3(kFusedWaves * 64), params,
                                    (unsigned)FShape<D>::launch_lds, stream);
}

template <int D>
hipError_t launch_fused_t(const FusedArgs& fa, int fp8, int erase, hipStream_t stream) {
  static DeviceOnce once;
  LaunchInfo li;
  const hipError_t ie = once.get([](int dev, LaunchInfo& info) {
    const void* fns[4] = {(const void*)gdn_fused_kernel<D, false, true>, (const void*)gdn_fused_kernel<D, false, false>,
                          (const void*)gdn_fused_kernel<D, true, true>, (const void*)gdn_fused_kernel<D, true, false>};
    hipError_t e = hipSuccess;
    int per_cu = 1 << 30;
    for (int i = 0; i < 4 && e == hipSuccess; ++i) {
      e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)FShape<D>::launch_lds);
      int occ = 0;
      if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fns[i], kFusedWaves * 64, FShape<D>::launch_lds);
      per_cu = occ < per_cu ? occ : per_cu;
    }
    if (e == hipSuccess) e = hipDeviceGetAttribute(&info.cus, hipDeviceAttributeMultiprocessorCount, dev);
    info.slots = per_cu == 2 ? 2 * info.cus : 0;                   // two workgroups per CU, exactly
    return e;
  }, &li);
  if (ie != hipSuccess) return ie;
  if (li.slots < 1) return hipErrorInvalidConfiguration;
  if (fa.grid > li.slots) return hipErrorInvalidConfiguration;
  const uint32_t words = (uint32_t)(fused_ctl_bytes(fa.BH) / 4);
  hipLaunchKernelGGL(gdn_fused_clear_kernel, dim3((words + 1023) / 1024 < 64 ? (words + 1023) / 1024 : 64),
                     dim3(1024), 0, stream, (uint32_t*)fa.ctl, words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (fp8) return erase ? launch_fused_t3<D, true, true>(fa, fa.grid, stream) : launch_fused_t3<D, true, false>(fa, fa.grid, stream);
  return erase ? launch_fused_t3<D, false, true>(fa, fa.grid, stream) : launch_fused_t3<D, false, false>(fa, fa.grid, stream);
}

// Static scratch of the allocation-free forward (gdn_frame_forward_noalloc):
// every GPU the library runs on holds its own copy until the process ends.
// Host code never passes the array's name to a kernel: its address on a
// device comes from hipGetSymbolAddress, taken once per device below.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;   // device -> address of that device's copy of `scratch`

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));   // with the device current: this device's copy
    if (e != hipSuccess) return e;
    if (!ptr || ((uintptr_t)ptr % 256) != 0) return hipErrorInvalidSymbol;
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return hipSuccess;
}

size_t fused_slot_bytes(int D) {
  const size_t nb = (size_t)D / 16;
  return (nb * (nb + 1) / 2 + 1) / 2 * 1024 + nb * nb * 512;
}

hipError_t launch_fused(int D, const FusedArgs& fa, int fp8, int erase, hipStream_t stream) {
  switch (D) {
    case 16: return launch_fused_t<16>(fa, fp8, erase, stream);
    case 32: return launch_fused_t<32>(fa, fp8, erase, stream);
    case 48: return launch_fused_t<48>(fa, fp8, erase, stream);
    case 64: return launch_fused_t<64>(fa, fp8, erase, stream);
    case 80: return launch_fused_t<80>(fa, fp8, erase, stream);
    case 96: return launch_fused_t<96>(fa, fp8, erase, stream);
    case 112: return launch_fused_t<112>(fa, fp8, erase, stream);
    case 128: return launch_fused_t<128>(fa, fp8, erase, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
