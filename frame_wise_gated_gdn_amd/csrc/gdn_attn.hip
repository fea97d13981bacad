// Block-causal softmax attention on gfx950 (the hybrid's periodic softmax
// blocks: SANA-WM keeps softmax attention blocks between its frame-wise GDN
// blocks, per the GeekNews summary of SANA-WM and the SANA-WM abstract).
//
//   O = softmax(Q K^T * scale) V   per (batch, head), tokens frame-major;
//   a query in frame f (of the key sequence; the queries are its last Tq
//   frames) sees the keys of every frame up to the end of its block of
//   `chunk` frames.
//
// One workgroup of eight waves owns 256 consecutive queries of one head and
// streams the visible keys and values through LDS in tiles of 64 tokens, one
// barrier per tile.  Each wave owns 32 queries.  Every key and value byte
// brought into a CU serves 256 queries: at 128 the kernel was bound by these
// re-reads (about 5 TB/s of K/V per call at the 720p clip).
//
// Each wave pipelines its own tiles: while it runs the softmax of key tile t
// it issues the score products of tile t+1, interleaved instruction by
// instruction (a second set of score registers), then the P V products of
// tile t.  Its VALU and matrix pipe work together, and the other wave on the
// SIMD fills what is left.
//
// Transposed formulation.  The wave computes S^T = K Q^T (keys as MFMA rows,
// queries as columns) and O^T = V^T P^T, so that in every accumulator a lane
// holds one query (column l%16) and four keys or four head-dim entries (rows
// 4g..4g+3):
//   * the online softmax state (running max m, running sum) is per lane, and
//     rescaling O by exp(m_old - m_new) needs no cross-lane traffic; the max
//     over a tile's keys takes two lane shuffles (the four lanes of a query),
//     and the sum is one more MFMA row block (bf16 ones times P^T), so the
//     denominator sums the same bf16 probabilities as the numerator;
//   * P goes from the S^T accumulators straight into the B operand of the
//     V^T P^T product (bf16), with the keys of a 32-key step taken in the
//     order 4g..4g+3, 16+4g..16+4g+3, which is the order in which the
//     transposing LDS read (ds_read_b64_tr_b16) hands each lane its column of
//     V; no LDS round trip for P.
//   * Q^T is the B operand of S^T: each lane loads its query row once, from
//     global memory, and keeps it in registers.
// Scores are scaled by scale*log2(e) (> 0) inside the exponent:
// p = exp2(s * scale*log2(e) - m).  Masked keys (past the query's block) score
// -inf; the running max starts finite, so no lane ever computes -inf - -inf.
//
// MFMA lane layouts are those of gdn_device.h (16x16x32 bf16).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kAttnWaves = 8;
constexpr int kAttnQW = 32;                        // queries per wave
constexpr int kAttnBM = kAttnWaves * kAttnQW;      // queries per workgroup
constexpr int kAttnBN = 64;                        // keys per tile

template <int D>
struct AttnShape {
  static constexpr int NB = D / 16;                // 16-wide head-dim blocks
  static constexpr int NKC = (D + 31) / 32;        // 32-wide k-steps of Q K^T
  static constexpr int NQ = kAttnQW / 16;          // query tiles per wave
  static constexpr int NKT = kAttnBN / 16;         // 16-key tiles per key tile
  static constexpr int NK2 = kAttnBN / 32;         // 32-key steps of V^T P^T
  static constexpr int UPR = D / 8;                // 16-byte units per token row
  static constexpr int UNITS = kAttnBN * UPR;      // units per K (or V) tile
  static constexpr int LPT = (UNITS + kAttnWaves * 64 - 1) / (kAttnWaves * 64);   // units per thread
  // LDS row strides (elements).  K rows are read 16 bytes per lane, eight
  // lanes (rows n..n+7) per pass: a stride of 112 modulo 128 bytes puts them
  // on distinct banks.  V rows are read by the transposing 8-byte read, four
  // rows of 32 bytes per 16 lanes: the stride must be 32 or 96 modulo 128
  // bytes (and eight rows distinct modulo 256).
  static constexpr int RS = D + 8;
  static constexpr int RSV = (D % 64 == 16 || D % 64 == 48) ? D : D + 16;
  static constexpr size_t tile_bytes = (size_t)kAttnBN * RS * 2;
  static constexpr size_t vtile_bytes = (size_t)kAttnBN * RSV * 2;
  static constexpr size_t lds_bytes = 3 * tile_bytes + 2 * vtile_bytes;   // K x 3 buffers, V x 2 buffers
};

__device__ __forceinline__ float wave_max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

// Keys visible to a query token qi of the query sequence (last Tq frames).
__device__ __forceinline__ int key_end(int qi, const AttnArgs& a) {
  const long long fq = (long long)(a.Tk - a.Tq) + qi / a.S;
  const long long end = (fq / a.chunk + 1) * (long long)a.chunk;   // any chunk up to INT_MAX
  return (int)(end < a.Tk ? end : (long long)a.Tk) * a.S;
}

template <int D>
__global__ __launch_bounds__(kAttnWaves * 64, 1) void gdn_attn_kernel(AttnArgs a) {
  using Sh = AttnShape<D>;
  constexpr int NB = Sh::NB, NKC = Sh::NKC, NQ = Sh::NQ, NKT = Sh::NKT, NK2 = Sh::NK2;
  constexpr int UPR = Sh::UPR, UNITS = Sh::UNITS, LPT = Sh::LPT, RS = Sh::RS, RSV = Sh::RSV;
  extern __shared__ __align__(16) unsigned char smem[];

  const int Nq = a.Tq * a.S, Nk = a.Tk * a.S;
  const int nqt = (Nq + kAttnBM - 1) / kAttnBM;
  // head-major; within a head the longest key ranges start first; the key
  // split part is innermost
  const int part = (int)(blockIdx.x % a.split), unit = (int)(blockIdx.x / a.split);
  const int bh = unit / nqt;
  const int qtile = nqt - 1 - unit % nqt;
  const int q0 = qtile * kAttnBM;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, n = l & 15, g = l >> 4;
  const uint16_t* qh = (const uint16_t*)a.q + (size_t)bh * Nq * D;
  const uint16_t* kh = (const uint16_t*)a.k + (size_t)bh * Nk * D;
  const uint16_t* vh = (const uint16_t*)a.v + (size_t)bh * Nk * D;
  uint16_t* oh = (uint16_t*)a.o + (size_t)bh * Nq * D;

  // the workgroup's key range: up to the block end of its last query, and of
  // that the tiles of this key-split part
  const int kend_wg = key_end(min(q0 + kAttnBM, Nq) - 1, a);
  const int ntiles = (kend_wg + kAttnBN - 1) / kAttnBN;
  const int tb = part * a.split_tiles;
  const int te = min(ntiles, tb + a.split_tiles);
  const int nt = max(0, te - tb);

  // this lane's queries (one per query tile) and their key ends; lane 0 holds
  // the wave's first query, whose key end is the wave's smallest
  int kend[NQ];
  u32x4 QB[NQ][NKC];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const int qi = q0 + kAttnQW * w + 16 * qt + n;
    kend[qt] = key_end(min(qi, Nq - 1), a);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int d = 32 * kc + 8 * g;
      QB[qt][kc] = (qi < Nq && d < D) ? *(const u32x4*)(qh + (size_t)qi * D + d) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const int kend_lo = __builtin_amdgcn_readfirstlane(kend[0]);
  f32x4 O[NQ][NB];
  float m[NQ];
  f32x4 L[NQ];                  // running sum of P per query (every row of a lane holds it)
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    m[qt] = -1e30f;
    L[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < NB; ++db) O[qt][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // K/V tile staging through registers.  A tile's rows are contiguous in HBM,
  // so unit u (16 bytes) sits 8u elements after the tile's first key; in LDS
  // the rows are padded to RS (K) or RSV (V) elements (offsets hoisted out of
  // the tile loop).
  u32x4 RK[LPT], RV[LPT];
  int lds_u[LPT], lds_v[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int u = tid + kAttnWaves * 64 * i;
    lds_u[i] = (u / UPR) * RS + 8 * (u % UPR);
    lds_v[i] = (u / UPR) * RSV + 8 * (u % UPR);
  }
  // buffer loads: a unit past the head's keys (or past the last tile) reads zeros
  const uint32_t head_bytes = (uint32_t)Nk * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kh, head_bytes), vrs = make_rsrc(vh, head_bytes);
  auto tile_off = [&](int t, int i) -> uint32_t {
    const int u = tid + kAttnWaves * 64 * i;
    return (u < UNITS && t < te) ? (uint32_t)t * kAttnBN * D * 2 + 16u * u : kOOB;
  };
  auto load_k = [&](int t) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) RK[i] = buf_load16_nt(krs, tile_off(t, i));
  };
  auto load_v = [&](int t) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) RV[i] = buf_load16_nt(vrs, tile_off(t, i));
  };
  // LDS: K buffers 0..2, then V buffers 0..1
  auto kbuf_ptr = [&](int b) { return (uint16_t*)(smem + (size_t)b * Sh::tile_bytes); };
  auto vbuf_ptr = [&](int b) { return (uint16_t*)(smem + 3 * Sh::tile_bytes + (size_t)b * Sh::vtile_bytes); };
  auto store_k = [&](int b) {
    uint16_t* dst = kbuf_ptr(b);
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      if (tid + kAttnWaves * 64 * i < UNITS) *(u32x4*)(dst + lds_u[i]) = RK[i];
  };
  auto store_v = [&](int b) {
    uint16_t* dst = vbuf_ptr(b);
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      if (tid + kAttnWaves * 64 * i < UNITS) *(u32x4*)(dst + lds_v[i]) = RV[i];
  };

  const float sl2 = a.scale_log2;
  // Scores of two key tiles live at once: Sx of the tile whose softmax runs
  // now, Sy of the next tile, whose products are issued in the same basic
  // block as the exponentials of Sx so that one wave keeps its matrix pipe
  // and its VALU busy together.
  f32x4 S0[NKT][NQ], S1[NKT][NQ];
  // S^T = K Q^T for one key tile: Sx[k16][qt], lane: query 16 qt + n, keys 16 k16 + 4 g + r
  auto scores = [&](const uint16_t* kt, f32x4 (&Sx)[NKT][NQ]) {
    u32x4 A[2][NKC];
    auto read_a = [&](int buf, int k16) {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const int d = 32 * kc + 8 * g;
        A[buf][kc] = d < D ? *(const u32x4*)(kt + (16 * k16 + n) * RS + d) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    read_a(0, 0);
#pragma unroll
    for (int k16 = 0; k16 < NKT; ++k16) {
      if (k16 + 1 < NKT) read_a((k16 + 1) & 1, k16 + 1);
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt) Sx[k16][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int qt = 0; qt < NQ; ++qt) Sx[k16][qt] = mfma_bf16(A[k16 & 1][kc], QB[qt][kc], Sx[k16][qt]);
    }
  };

  // One key tile t (keys from kb): softmax of Sx, the next tile's scores into
  // Sy (from the K tile at ktn), then O += V^T P^T with the tile's V (vt).
  auto tile = [&](int kb, const uint16_t* vt, const uint16_t* ktn, f32x4 (&Sx)[NKT][NQ],
                  f32x4 (&Sy)[NKT][NQ]) {
    if (kb + kAttnBN > kend_lo) {
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
        for (int k16 = 0; k16 < NKT; ++k16)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kb + 16 * k16 + 4 * g + r >= kend[qt]) Sx[k16][qt][r] = -INFINITY;
    }
    float mold[NQ], mnew[NQ];
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int k16 = 0; k16 < NKT; ++k16)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, Sx[k16][qt][r]);
      mx = wave_max4(mx);
      mold[qt] = m[qt];
      mnew[qt] = fmaxf(mold[qt], mx * sl2);
      m[qt] = mnew[qt];
    }
    // rescale before the products of the next tile, so that they, the
    // exponentials and P V share one basic block
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt) {
      if (__any(mnew[qt] > mold[qt])) {
        const float alpha = __builtin_amdgcn_exp2f(mold[qt] - mnew[qt]);
        L[qt] *= alpha;
#pragma unroll
        for (int db = 0; db < NB; ++db) O[qt][db] *= alpha;
      }
    }
    scores(ktn, Sy);
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
      for (int k16 = 0; k16 < NKT; ++k16)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Sx[k16][qt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(Sx[k16][qt][r], sl2, -mnew[qt]));
    // issue order: each product of the next tile followed by VALU
    // instructions of this tile's exponentials (an fma and an exp per score),
    // so the wave issues VALU work while its products run
    constexpr int NSC = NKT * NKC * NQ;                  // products of one tile's scores
    constexpr int VPS = (2 * NKT * 4 * NQ + NSC - 1) / NSC;
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, VPS, 0); // then VPS VALU instructions
    }
    u32x4 PB[NQ][NK2];
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
      for (int k2 = 0; k2 < NK2; ++k2) {
        const f32x4 lo = Sx[2 * k2][qt], hi = Sx[2 * k2 + 1][qt];
        PB[qt][k2] = u32x4{pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]), pack_bf16(hi[0], hi[1]),
                           pack_bf16(hi[2], hi[3])};
      }
    // A operand = V columns 16 db + n at keys 32 k2 + {4g..4g+3, 16+4g..16+4g+3};
    // the next column block's operands are read while the current one's run
    u32x4 VA[2][NK2];
    auto read_v = [&](int buf, int db) {
#pragma unroll
      for (int k2 = 0; k2 < NK2; ++k2) {
        const uint16_t* p0 = vt + (32 * k2 + 4 * g + (n >> 2)) * RSV + 16 * db + 4 * (n & 3);
        const u32x2 x = lds_tr16(p0), y = lds_tr16(p0 + 16 * RSV);
        VA[buf][k2] = u32x4{x[0], x[1], y[0], y[1]};
      }
    };
    read_v(0, 0);
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      if (db + 1 < NB) read_v((db + 1) & 1, db + 1);
#pragma unroll
      for (int k2 = 0; k2 < NK2; ++k2)
#pragma unroll
        for (int qt = 0; qt < NQ; ++qt) O[qt][db] = mfma_bf16(VA[db & 1][k2], PB[qt][k2], O[qt][db]);
    }
    const u32x4 ONES = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
#pragma unroll
    for (int k2 = 0; k2 < NK2; ++k2)
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt) L[qt] = mfma_bf16(ONES, PB[qt][k2], L[qt]);
  };

  // At the top of iteration t the LDS holds K tiles t and t+1 and V tile t;
  // the wave holds the scores of tile t.  Iteration t stores K tile t+2
  // (buffer (t+2)%3, last read in iteration t-1) and V tile t+1 (buffer
  // (t+1)%2, last read in iteration t-1), then prefetches K t+3 and V t+2.
  // Past the last tile the loads read zeros and the stores stage them, so the
  // next-tile scores of the last iteration (never used) read defined LDS.
  load_k(tb);
  load_v(tb);
  store_k(0);
  store_v(0);
  load_k(tb + 1);
  store_k(1);
  load_k(tb + 2);
  load_v(tb + 1);
  lds_barrier();
  if (nt > 0) scores(kbuf_ptr(0), S0);
  int kb1 = 1, kb2 = 2;                   // K buffers of tiles t+1, t+2
  auto iteration = [&](int it, f32x4 (&Sx)[NKT][NQ], f32x4 (&Sy)[NKT][NQ]) {
    const int t = tb + it;
    lds_barrier();
    tile(t * kAttnBN, vbuf_ptr(it & 1), kbuf_ptr(kb1), Sx, Sy);
    store_k(kb2);
    store_v((it + 1) & 1);
    load_k(t + 3);
    load_v(t + 2);
    const int kfree = 3 - kb1 - kb2;      // buffer of tile t, free after this iteration
    kb1 = kb2;
    kb2 = kfree;
  };
  for (int it = 0; it < nt; it += 2) {
    iteration(it, S0, S1);
    if (it + 1 < nt) iteration(it + 1, S1, S0);
  }
  // lane holds O[query 16 qt + n][16 db + 4 g + r]
  if (a.split > 1) {
    // partial state of this key range: unnormalised O, running max and sum
    const size_t prow = ((size_t)part * a.BH + bh) * Nq;
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt) {
      const int qi = q0 + kAttnQW * w + 16 * qt + n;
      if (qi < Nq) {
#pragma unroll
        for (int db = 0; db < NB; ++db)
          *(f32x4*)(a.part_o + (prow + qi) * D + 16 * db + 4 * g) = O[qt][db];
        if (g == 0) *(f32x2*)(a.part_ml + (prow + qi) * 2) = f32x2{m[qt], L[qt][0]};
      }
    }
    return;
  }
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const int qi = q0 + kAttnQW * w + 16 * qt + n;
    const float inv = 1.f / L[qt][0];
    if (qi < Nq) {
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        const f32x4 x = O[qt][db] * inv;
        *(u32x2*)(oh + (size_t)qi * D + 16 * db + 4 * g) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
      }
    }
  }
}

// Merge of the key-split partial states, one thread per (head, query, eight
// head-dim entries): O = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) L_p with
// M = max_p m_p, in a fixed order of the parts.
__global__ __launch_bounds__(256) void gdn_attn_merge_kernel(AttnArgs a, int D) {
  const int Nq = a.Tq * a.S, G8 = D / 8;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)a.BH * Nq * G8) return;
  const long long row = idx / G8;                     // bh * Nq + qi
  const int d0 = (int)(idx % G8) * 8;
  const size_t stride = (size_t)a.BH * Nq;
  float M = -INFINITY;
  for (int p = 0; p < a.split; ++p) M = fmaxf(M, a.part_ml[(p * stride + row) * 2]);
  float den = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < a.split; ++p) {
    const f32x2 ml = *(const f32x2*)(a.part_ml + (p * stride + row) * 2);
    const float wgt = __builtin_amdgcn_exp2f(ml[0] - M);
    den = __builtin_fmaf(wgt, ml[1], den);
    const f32x4* src = (const f32x4*)(a.part_o + (p * stride + row) * D + d0);
    const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = __builtin_fmaf(wgt, x0[i], acc[i]);
      acc[4 + i] = __builtin_fmaf(wgt, x1[i], acc[4 + i]);
    }
  }
  const float inv = 1.f / den;
  *(u32x4*)((uint16_t*)a.o + row * D + d0) =
      u32x4{pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv),
            pack_bf16(acc[4] * inv, acc[5] * inv), pack_bf16(acc[6] * inv, acc[7] * inv)};
}

template <int D>
hipError_t launch_attn_t(const AttnArgs& a, hipStream_t stream) {
  using Sh = AttnShape<D>;
  const long long Nq = (long long)a.Tq * a.S;
  const long long nqt = (Nq + kAttnBM - 1) / kAttnBM;
  const long long blocks = nqt * a.BH * a.split;
  if (blocks > 0x7fffffffLL || a.split < 1) return hipErrorInvalidConfiguration;
  static DeviceOnce once;
  LaunchInfo li;
  const hipError_t ie = once.get([](int, LaunchInfo&) {
    return hipFuncSetAttribute((const void*)gdn_attn_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)Sh::lds_bytes);
  }, &li);
  if (ie != hipSuccess) return ie;
  hipLaunchKernelGGL(gdn_attn_kernel<D>, dim3((unsigned)blocks), dim3(kAttnWaves * 64), Sh::lds_bytes, stream, a);
  if (a.split > 1) {
    const long long threads = (long long)a.BH * Nq * (D / 8);
    hipLaunchKernelGGL(gdn_attn_merge_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a, D);
  }
  return hipGetLastError();
}

}  // namespace

// Key tiles of the longest workgroup of a launch (its last query's block end).
static long long attn_max_tiles(int Tq, int Tk, int S, int chunk) {
  const long long Nq = (long long)Tq * S;
  const long long fq = (long long)(Tk - Tq) + (Nq - 1) / S;
  const long long kend = std::min<long long>(Tk, (fq / chunk + 1) * (long long)chunk) * S;
  return (kend + kAttnBN - 1) / kAttnBN;
}

int attn_split_parts(int D, int BH, int Tq, int Tk, int S, int chunk, int cus) {
  (void)D;
  const long long Nq = (long long)Tq * S;
  const long long units = (Nq + kAttnBM - 1) / kAttnBM * BH;        // workgroups without a split
  const long long tiles = attn_max_tiles(Tq, Tk, S, chunk);
  // one workgroup per CU at a time: pick the part count with the fewest
  // rounds of workgroups per unit of work, at least 8 key tiles per part
  int best = 1;
  double best_cost = (double)((units + cus - 1) / cus);
  for (int p = 2; p <= 8; ++p) {
    if (tiles < 8LL * p) break;
    const double cost = (double)((units * p + cus - 1) / cus) / p;
    if (cost < 0.9 * best_cost) {
      best = p;
      best_cost = cost;
    }
  }
  return best;
}

int attn_split_tiles(int Tq, int Tk, int S, int chunk, int parts) {
  const long long tiles = attn_max_tiles(Tq, Tk, S, chunk);
  return (int)((tiles + parts - 1) / parts);
}

size_t attn_split_bytes(int D, int BH, int Tq, int S, int parts) {
  if (parts <= 1) return 0;
  const size_t rows = (size_t)parts * BH * Tq * S;
  return rows * D * 4 + ((rows * 2 * 4 + 255) & ~(size_t)255);
}

hipError_t launch_attn(int D, const AttnArgs& a, hipStream_t stream) {
  switch (D) {
    case 16: return launch_attn_t<16>(a, stream);
    case 32: return launch_attn_t<32>(a, stream);
    case 48: return launch_attn_t<48>(a, stream);
    case 64: return launch_attn_t<64>(a, stream);
    case 80: return launch_attn_t<80>(a, stream);
    case 96: return launch_attn_t<96>(a, stream);
    case 112: return launch_attn_t<112>(a, stream);
    case 128: return launch_attn_t<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
