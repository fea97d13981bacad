// Frame-wise Gated DeltaNet forward: CDNA4 (gfx950) kernels.
//
// The recurrence (SANA-WM news article "NVIDIA Apresenta SANA-WM ...", section
// "1. Atencao Linear Hibrida com Gated DeltaNet (GDN)"): per head a D x D state
// M[key][value] is carried across frames; frame t of S tokens does
//   Md = g_t M;  P = Kf Md;  R = V - b_t P (ERASE) or b_t (V - P) (WRITE);
//   M = Md + Kf^T R;  O_t = Qf M,   Kf = ReLU(K)/sqrt(D*S), Qf = ReLU(Q).
//
// This file holds the single-pass recurrence (fp32 I/O always; bf16 I/O with
// GDN_FLAG_DIRECT) and the two readouts; the default bf16 path computes the
// states with the Gram pipeline of gdn_gram.hip and then reads them out here.
//
// Single-pass recurrence: one workgroup per (head, 16-wide value-column tile
// of M).  Columns of M evolve independently (each column only meets the same
// column of V, R and O), so the tile's state lives in registers for the whole
// frame loop.  The 8 waves of the workgroup split the frame's tokens into
// chunks; per chunk a wave runs the prediction (MFMA against the copy of M),
// the residual, and the write Kf^T R (MFMA; in bf16 the residual is split
// into a hi+lo pair so that the write keeps ~16 bits).  The waves' partial
// writes are reduced through LDS in fixed order (deterministic), the owning
// wave updates its 16-key block of M in fp32, and the new M is published to
// LDS for the next frame and to a per-frame snapshot in HBM.  Workgroups of
// one head are placed on the same XCD (workgroups are dealt to the 8 XCDs
// round-robin by id), so the re-reads of a frame's keys by the head's column
// tiles hit that XCD's L2.
//
// Readout: O_t = Qf M_t for every frame in parallel from the snapshots
// (HBM-bound), plus the optional state norms.
//
// MFMA and LDS lane layouts are listed in gdn_device.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kWaves = 8;          // waves per recurrence workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kReadWaves = 4;      // waves per readout workgroup

// ----------------------------------------------------------------------------
// fp32 recurrence (fp32 I/O).  One workgroup per (head, 16-wide value tile);
// the 8 waves split the frame's tokens in 16-token chunks; per chunk a wave
// runs the prediction and the write with v_mfma_f32_16x16x4_f32 (the k index
// of MFMA step kc on lane group g is key g*(D/4)+kc), the waves' partial
// writes are reduced through LDS in fixed order, and the owning wave updates
// its 16-key block of the tile in fp32.
// ----------------------------------------------------------------------------
template <int D>
struct RecurShapeF32 {
  static constexpr int NB = D / 16;                      // key blocks == value tiles
  static constexpr int TOK = 16;                         // tokens per wave chunk
  static constexpr int KS = D + 4;                       // ReLU(K) staging row stride (elements)
  static constexpr int MBS = D + 4;                      // mbT row stride
  static constexpr size_t kst_bytes = (size_t)kWaves * TOK * KS * 4;
  static constexpr size_t red_bytes = (size_t)kWaves * NB * 64 * 16;
  static constexpr size_t mbt_bytes = (size_t)16 * MBS * 4;
  static constexpr size_t lds_bytes = kst_bytes + red_bytes + mbt_bytes + 64;
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void gdn_recur_f32_kernel(RecurArgs a) {
  using Sh = RecurShapeF32<D>;
  constexpr int NB = Sh::NB, TOK = Sh::TOK, KS = Sh::KS, MBS = Sh::MBS;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* kst_base = smem;
  f32x4* red = (f32x4*)(smem + Sh::kst_bytes);
  unsigned char* mbt = smem + Sh::kst_bytes + Sh::red_bytes;
  float* normp = (float*)(mbt + Sh::mbt_bytes);

  const int unit = xcd_unit(a.units);
  if (unit < 0) return;                       // whole workgroup leaves together
  const int bh = unit / NB, jt = unit % NB, j0 = jt * 16;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), g = l >> 4, n = l & 15;
  const int S = a.S, T = a.T;
  const size_t head_off = (size_t)bh * T * S * D;     // element offset of this head
  const float c = a.kscale;
  const bool erase = a.beta_mode == 0;

  // ---- initial state: wave w < NB owns key rows 16w..16w+15 of the tile (C layout)
  f32x4 Mown = {0.f, 0.f, 0.f, 0.f};
  if (w < NB && a.state_src) {
    const float* src = a.state_src + (size_t)bh * D * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) Mown[i] = src[(size_t)(16 * w + 4 * g + i) * D + j0 + n];
  }
  // zero mbT (including the padding), then publish M0
  for (int x = tid; x < (int)(Sh::mbt_bytes / 4); x += kThreads) ((uint32_t*)mbt)[x] = 0u;
  __syncthreads();
  if (w < NB) {
    float* mb = (float*)mbt;
#pragma unroll
    for (int i = 0; i < 4; ++i) mb[n * MBS + 16 * w + 4 * g + i] = Mown[i];
  }
  __syncthreads();

  // B operand of the prediction: value column n, keys g*(D/4)+kc, loaded
  // from mbT after every frame.
  float MBf[D / 4];
  auto load_mb = [&]() {
    const float* mb = (const float*)mbt;
#pragma unroll
    for (int kc = 0; kc < D / 4; ++kc) MBf[kc] = mb[n * MBS + g * (D / 4) + kc];
  };
  load_mb();

  const int nchunks = (S + TOK - 1) / TOK;
  const float* kf32 = (const float*)a.k + head_off;
  const float* vf32 = (const float*)a.v + head_off;

  for (int tl = 0; tl < a.Tc; ++tl) {
    const int t = a.t0 + tl;
    const float gam = a.gamma[(size_t)bh * T + t];
    const float bet = a.beta[(size_t)bh * T + t];
    const float s_pred = bet * c * gam;        // R = av*V - s_pred * (phi(K) M)
    const float av = erase ? 1.0f : bet;
    const size_t fo = (size_t)t * S * D;       // frame offset inside the head

    f32x4 Wacc[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) Wacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int ch = w; ch < nchunks; ch += kWaves) {
      const int tb = ch * TOK;
      {
        float* kst = (float*)kst_base + (size_t)w * TOK * KS;
        // -- loads: ReLU(K) rows, lane (token n, keys g*(D/4) .. +D/4-1)
        const int tok = tb + n;
        float KAf[D / 4];
#pragma unroll
        for (int kc = 0; kc < D / 4; ++kc) {
          const float x = (tok < S) ? kf32[fo + (size_t)tok * D + g * (D / 4) + kc] : 0.f;
          KAf[kc] = x > 0.f ? x : 0.f;
        }
#pragma unroll
        for (int kc = 0; kc < D / 4; ++kc) kst[n * KS + g * (D / 4) + kc] = KAf[kc];
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < D / 4; ++kc) P = mfma_f32(KAf[kc], MBf[kc], P);
        wave_lds_sync();
        float R[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = tb + 4 * g + i;
          const float vv = (tk < S) ? vf32[fo + (size_t)tk * D + j0 + n] : 0.f;
          R[i] = av * vv - s_pred * P[i];
        }
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            Wacc[kb] = mfma_f32(kst[(4 * g + i) * KS + 16 * kb + n], R[i], Wacc[kb]);
        wave_lds_sync();
      }
    }

    // ---- reduce the waves' partial writes (fixed order), update the owned block
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) red[(w * NB + kb) * 64 + l] = Wacc[kb];
    __syncthreads();
    if (w < NB) {
      f32x4 s = red[w * 64 + l];
      for (int ww = 1; ww < kWaves; ++ww) {
        const f32x4 x = red[(ww * NB + w) * 64 + l];
        s[0] += x[0]; s[1] += x[1]; s[2] += x[2]; s[3] += x[3];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Mown[i] = gam * Mown[i] + c * s[i];
      // publish M to mbT and to the frame snapshot (transposed: row = value
      // column, contiguous keys)
      const size_t snap_off = ((size_t)bh * a.Tc + tl) * D * D + (size_t)(j0 + n) * D + 16 * w + 4 * g;
      float* mb = (float*)mbt;
#pragma unroll
      for (int i = 0; i < 4; ++i) mb[n * MBS + 16 * w + 4 * g + i] = Mown[i];
      *(f32x4*)((float*)a.snap + snap_off) = Mown;
      if (a.norm_part) {
        float sq = Mown[0] * Mown[0] + Mown[1] * Mown[1] + Mown[2] * Mown[2] + Mown[3] * Mown[3];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off, 64);
        if (l == 0) normp[w] = sq;
      }
    }
    __syncthreads();
    load_mb();
    if (a.norm_part && tid == 0) {
      float sq = 0.f;
      for (int kb = 0; kb < NB; ++kb) sq += normp[kb];
      a.norm_part[((size_t)bh * a.Tc + tl) * NB + jt] = sq;
    }
  }

  if (w < NB && a.state_dst) {
    float* dst = a.state_dst + (size_t)bh * D * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(size_t)(16 * w + 4 * g + i) * D + j0 + n] = Mown[i];
  }
}

// ----------------------------------------------------------------------------
// bf16 recurrence with a register ring of prefetched chunks.
//
// Each wave walks the flattened sequence of its (frame, chunk) slots; slot s
// uses register buffer s % kRing, and the loads of slot s + kRing are issued
// right after slot s is consumed, so every chunk's keys and values are in
// flight for kRing slots (one whole frame when a frame has kRing slots per
// wave).  Nothing in a load depends on the state, so this prefetch crosses
// frame boundaries freely.  The loads are buffer loads whose out-of-range
// lanes (tokens past S, keys past D, chunks past the frame) are given an
// offset beyond the buffer and so read zeros without touching memory: the
// loads are branch-free and always issued, which keeps the wait counts exact.
// The per-frame barriers only wait for LDS traffic, never for the prefetches.
// ----------------------------------------------------------------------------
constexpr int kRing = 4;

// The values enter the prediction MFMA as extra k-slots: the A operand of the
// last k-chunk carries the 16 value columns of the tile in lanes g = 2, 3 and
// the B operand holds -I there, so the MFMA returns P' = phi(K) bf16(s M) - V
// = -R directly (s = beta c gamma for ERASE, c gamma for WRITE).  For D = 16
// mod 32 these slots are the free half of the last key chunk; otherwise one
// extra chunk is added.
template <int D>
struct BfShape {
  static constexpr int NB = D / 16;
  static constexpr int NKK = (D + 31) / 32;              // k-chunks holding keys
  static constexpr bool VIN = (D % 32) == 16;            // values fit in the last key chunk
  static constexpr int NKC = VIN ? NKK : NKK + 1;        // k-chunks of the prediction
  static constexpr int UPR = D / 8;                      // 16-byte units per token row
  static constexpr int NLD = D / 16;                     // 1 KB key loads per 32-token chunk
  static constexpr int KS = D + 8;                       // LDS key row stride (elements)
  static constexpr int MBS = 32 * NKC + 8;               // LDS B-operand row stride (elements)
  static constexpr size_t kst_bytes = (size_t)kWaves * 32 * KS * 2;
  static constexpr size_t red_bytes = (size_t)kWaves * NB * 64 * 16;
  static constexpr size_t mbt_bytes = (size_t)16 * MBS * 2;
  static constexpr size_t gb_bytes = (size_t)kMaxFramesPerLaunch * 8;
  static constexpr size_t lds_bytes = kst_bytes + red_bytes + mbt_bytes + 64 + gb_bytes;
};

template <int D, bool ERASE>
__global__ __launch_bounds__(kThreads, 1) void gdn_recur_bf16_kernel(RecurArgs a) {
  using Sh = BfShape<D>;
  constexpr int NB = Sh::NB, NKC = Sh::NKC, UPR = Sh::UPR, NLD = Sh::NLD, KS = Sh::KS, MBS = Sh::MBS;
  constexpr bool VIN = Sh::VIN;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
  uint16_t* const kst = (uint16_t*)smem + (size_t)w * 32 * KS;
  f32x4* const red = (f32x4*)(smem + Sh::kst_bytes);
  uint16_t* const mbt = (uint16_t*)(smem + Sh::kst_bytes + Sh::red_bytes);
  float* const normp = (float*)(smem + Sh::kst_bytes + Sh::red_bytes + Sh::mbt_bytes);
  float2* const gb = (float2*)(smem + Sh::kst_bytes + Sh::red_bytes + Sh::mbt_bytes + 64);

  const int unit = xcd_unit(a.units);
  if (unit < 0) return;                       // whole workgroup leaves together
  const int bh = unit / NB, jt = unit % NB, j0 = jt * 16;
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, n = l & 15;
  const int S = a.S, T = a.T;
  const float c = a.kscale;
  const uint32_t head_bytes = (uint32_t)T * (uint32_t)S * D * 2u;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc((const uint16_t*)a.k + (size_t)bh * T * S * D, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const uint16_t*)a.v + (size_t)bh * T * S * D, head_bytes);
  // snapshots and norm partials of this head only: byte offsets within a
  // head stay far below the out-of-range marker whatever B*H is
  const __amdgpu_buffer_rsrc_t snaprs =
      make_rsrc((unsigned char*)a.snap + (size_t)bh * a.Tc * D * D * 2, (uint32_t)((size_t)a.Tc * D * D * 2));
  const __amdgpu_buffer_rsrc_t normrs =
      make_rsrc(a.norm_part ? (unsigned char*)a.norm_part + (size_t)bh * a.Tc * NB * 4 : nullptr,
                a.norm_part ? (uint32_t)((size_t)a.Tc * NB * 4) : 0u);

  for (int x = tid; x < a.Tc; x += kThreads)
    gb[x] = make_float2(a.gamma[(size_t)bh * T + a.t0 + x], a.beta[(size_t)bh * T + a.t0 + x]);
  // ---- initial state: wave w < NB owns key rows 16w..16w+15 of the tile (C layout)
  f32x4 Mown = {0.f, 0.f, 0.f, 0.f};
  if (w < NB && a.state_src) {
    const float* src = a.state_src + (size_t)bh * D * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) Mown[i] = src[(size_t)(16 * w + 4 * g + i) * D + j0 + n];
  }
  // B operand rows: keys (filled per frame) and -I on the value slots
  for (int x = tid; x < (int)(Sh::mbt_bytes / 4); x += kThreads) ((uint32_t*)mbt)[x] = 0u;
  __syncthreads();
  if (tid < 16) mbt[tid * MBS + 32 * (NKC - 1) + 16 + tid] = 0xBF80u;   // bf16(-1)
  // scale of the state inside the prediction for frame tl
  auto pred_scale = [&](int tl) {
    const float2 x = gb[tl];
    return ERASE ? x.y * c * x.x : c * x.x;
  };
  if (w < NB) {
    const float s0 = pred_scale(0);
    const u32x2 pk = {pack_bf16(s0 * Mown[0], s0 * Mown[1]), pack_bf16(s0 * Mown[2], s0 * Mown[3])};
    *(u32x2*)(mbt + n * MBS + 16 * w + 4 * g) = pk;
  }
  __syncthreads();
  u32x4 MB[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) MB[kc] = *(const u32x4*)(mbt + n * MBS + 32 * kc + 8 * g);

  const int nchunks = (S + 31) / 32;
  const int NS = (nchunks + kWaves - 1) / kWaves;    // chunk slots per wave per frame
  const uint32_t frame_bytes = (uint32_t)S * D * 2u;
  // per-lane byte offsets of the value columns (lanes g >= 2) inside a chunk
  const uint32_t voff0 = (uint32_t)(n * D + j0 + 8 * (g & 1)) * 2u;
  const uint32_t voff1 = voff0 + 16u * D * 2u;

  // ---- A slot is (frame tl, chunk slot i): the wave's chunk w + kWaves*i of
  // frame tl.  Loads are branch-free: a null slot gets an offset past the
  // buffer (a uniform select; offsets added to it stay past the buffer), rows
  // past the frame are cleared when the chunk is used, reads past the head
  // read zeros.
  auto chunk_base = [&](int tl, int i) -> uint32_t {
    const int ch = w + kWaves * i;
    return (ch < nchunks && tl < a.Tc) ? (uint32_t)(a.t0 + tl) * frame_bytes + (uint32_t)ch * (64u * D) : kOOB;
  };
  auto load_k = [&](int tl, int i, u32x4 (&KU)[NLD]) {
    const uint32_t cb = chunk_base(tl, i);
#pragma unroll
    for (int j = 0; j < NLD; ++j) KU[j] = buf_load16(krs, cb + 16u * l + 1024u * j);
  };
  auto load_v = [&](int tl, int i, u32x4 (&VV)[2]) {
    const uint32_t cb = chunk_base(tl, i);
    VV[0] = buf_load16(vrs, g >= 2 ? cb + voff0 : kOOB);
    VV[1] = buf_load16(vrs, g >= 2 ? cb + voff1 : kOOB);
  };

  f32x4 Wacc[NB];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) Wacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- stage a chunk's keys: ReLU, then the wave's LDS tile (row-major,
  // padded).  Lanes exchange data through this tile: LDS operations of one
  // wave execute in program order, and the compiler keeps that order because
  // the addresses are lane-dependent (may alias).
  auto stage = [&](int tl, int i, u32x4 (&KU)[NLD]) {
    const int ch = w + kWaves * i;
    if (ch >= nchunks || tl >= a.Tc) return;   // wave-uniform
    const int lim = S - ch * 32;               // valid rows of the chunk
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int u = 64 * j + l;
      u32x4 x = relu8(KU[j]);
      if (lim < 32 && u / UPR >= lim) x = u32x4{0u, 0u, 0u, 0u};   // ragged last chunk
      *(u32x4*)(kst + (u / UPR) * KS + 8 * (u % UPR)) = x;
    }
  };

  // ---- one staged chunk: P' = -R from the MFMA, its hi/lo split, write accumulation
  auto compute = [&](int tl, int i, const u32x4 (&VV)[2]) {
    const int ch = w + kWaves * i;
    if (ch >= nchunks || tl >= a.Tc) return;   // wave-uniform
    const int lim = S - ch * 32;
    f32x4 P[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      P[r] = f32x4{0.f, 0.f, 0.f, 0.f};
      const u32x4 vr = (16 * r + n < lim) ? VV[r] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        u32x4 A;
        if (kc < NKC - 1) {
          A = *(const u32x4*)(kst + (16 * r + n) * KS + 32 * kc + 8 * g);
        } else if constexpr (VIN) {
          const u32x4 kk = *(const u32x4*)(kst + (16 * r + n) * KS + 32 * kc + 8 * (g & 1));
          A = (g >= 2) ? vr : kk;
        } else {
          A = (g >= 2) ? vr : u32x4{0u, 0u, 0u, 0u};
        }
        P[r] = mfma_bf16(A, MB[kc], P[r]);
      }
    }
    // P' = -R: split into bf16 hi + lo for the write's B operand
    u32x4 RBhi, RBlo;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint32_t h01 = pack_bf16(P[r][0], P[r][1]), h23 = pack_bf16(P[r][2], P[r][3]);
      RBhi[2 * r] = h01;
      RBhi[2 * r + 1] = h23;
      RBlo[2 * r] = pack_bf16(P[r][0] - bf16_lo_f32(h01), P[r][1] - bf16_hi_f32(h01));
      RBlo[2 * r + 1] = pack_bf16(P[r][2] - bf16_lo_f32(h23), P[r][3] - bf16_hi_f32(h23));
    }
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      const uint16_t* p0 = kst + (4 * g + (n >> 2)) * KS + 16 * kb + 4 * (n & 3);
      const u32x2 a0 = lds_tr16(p0);
      const u32x2 a1 = lds_tr16(p0 + 16 * KS);
      const u32x4 A = {a0[0], a0[1], a1[0], a1[1]};
      Wacc[kb] = mfma_bf16(A, RBhi, Wacc[kb]);
      Wacc[kb] = mfma_bf16(A, RBlo, Wacc[kb]);
    }
  };

  // ---- end of a frame: reduce the waves' partial writes (fixed order), update
  // the owned 16-key block (M = gamma M + c alpha Kf^T R, alpha = 1 or beta),
  // publish bf16(M) to the snapshot and bf16(s' M) to LDS for the next frame.
  auto end_frame = [&](int tl) {
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) red[(w * NB + kb) * 64 + l] = Wacc[kb];
    lds_barrier();
    // waves w >= NB run the same instructions on a clamped block and drop
    // their stores, so every wave issues the same memory operations
    const int ob = w < NB ? w : NB - 1;
    f32x4 sum = red[ob * 64 + l];
    for (int ww = 1; ww < kWaves; ++ww) {
      const f32x4 x = red[(ww * NB + ob) * 64 + l];
      sum[0] += x[0]; sum[1] += x[1]; sum[2] += x[2]; sum[3] += x[3];
    }
    const float2 gbt = gb[tl];
    const float upd = ERASE ? c : c * gbt.y;        // sum accumulated -R
    f32x4 Mn;
#pragma unroll
    for (int i = 0; i < 4; ++i) Mn[i] = gbt.x * Mown[i] - upd * sum[i];
    if (w < NB) Mown = Mn;
    const u32x2 pk = {pack_bf16(Mn[0], Mn[1]), pack_bf16(Mn[2], Mn[3])};
    const uint32_t snap_off = (uint32_t)((size_t)tl * D * D * 2 + (size_t)((jt * NB + ob) * 64 + l) * 8);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pk), snaprs, w < NB ? snap_off : kOOB, 0, 0);
    const float s1 = pred_scale(tl + 1 < a.Tc ? tl + 1 : tl);
    const u32x2 pm = {pack_bf16(s1 * Mn[0], s1 * Mn[1]), pack_bf16(s1 * Mn[2], s1 * Mn[3])};
    if (w < NB) *(u32x2*)(mbt + n * MBS + 16 * w + 4 * g) = pm;
    if (a.norm_part) {
      float sq = Mn[0] * Mn[0] + Mn[1] * Mn[1] + Mn[2] * Mn[2] + Mn[3] * Mn[3];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off, 64);
      if (w < NB && l == 0) normp[w] = sq;
    }
    lds_barrier();
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) MB[kc] = *(const u32x4*)(mbt + n * MBS + 32 * kc + 8 * g);
    if (a.norm_part) {
      float sq = 0.f;
      for (int kb = 0; kb < NB; ++kb) sq += normp[kb];
      const uint32_t noff = (uint32_t)(((size_t)tl * NB + jt) * 4);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sq), normrs, tid == 0 ? noff : kOOB, 0, 0);
    }
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) Wacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // Software pipeline over the wave's slots (s = 0, 1, ...): iteration s
  // computes slot s from the staged LDS tile and the values loaded kRing slots
  // earlier, then stages slot s + 1 (its ReLU and LDS writes overlap the MFMAs
  // of slot s), and refills the two register rings: values of slot s + kRing,
  // keys of slot s + 1 + kRing.  Slots past the last frame are null: their
  // loads read zeros without touching memory, so every ring load is issued
  // unconditionally and each wait count is exact.  The prologue issues its
  // loads in the loop's order (keys s+1 after values s) for the same reason.
  u32x4 KU[kRing][NLD];
  u32x4 VV[kRing][2];
  int ktl = 0, ki = 0;                       // next slot whose keys are loaded
  int vtl = 0, vi = 0;                       // next slot whose values are loaded
  auto advance = [&](int& tl, int& i) {
    if (++i == NS) { i = 0; ++tl; }
  };
  load_k(ktl, ki, KU[0]);
  advance(ktl, ki);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < kRing; ++r) {
    load_v(vtl, vi, VV[r]);
    advance(vtl, vi);
    __builtin_amdgcn_sched_barrier(0);
    if (r + 1 < kRing) {
      load_k(ktl, ki, KU[r + 1]);
      advance(ktl, ki);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  stage(0, 0, KU[0]);
  load_k(ktl, ki, KU[0]);
  advance(ktl, ki);
  __builtin_amdgcn_sched_barrier(0);
  int ptl = 0, pi = 0;                       // slot being computed
  int qtl = 0, qi = 0;                       // slot to stage next (= computed + 1)
  advance(qtl, qi);
  while (ptl < a.Tc) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      compute(ptl, pi, VV[r]);
      load_v(vtl, vi, VV[r]);
      advance(vtl, vi);
      stage(qtl, qi, KU[(r + 1) % kRing]);
      load_k(ktl, ki, KU[(r + 1) % kRing]);
      advance(ktl, ki);
      // keep the prefetch loads where they are issued (the scheduler would
      // otherwise sink them towards their use); other work may move across
      __builtin_amdgcn_sched_barrier(0x78F);
      if (pi == NS - 1 && ptl < a.Tc) end_frame(ptl);
      advance(ptl, pi);
      advance(qtl, qi);
    }
  }

  if (w < NB && a.state_dst) {
    float* dst = a.state_dst + (size_t)bh * D * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(size_t)(16 * w + 4 * g + i) * D + j0 + n] = Mown[i];
  }
}

// ----------------------------------------------------------------------------
// fp32 readout: O_t = Qf M_t, computed as O^T = M^T Qf^T so that each lane
// stores 4 consecutive output columns of one token; M_t^T is staged in LDS.
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kReadWaves * 64) void gdn_readout_f32_kernel(ReadoutArgs a) {
  constexpr int NB = D / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int frame = blockIdx.x;                    // over BH * Tc
  const int bh = frame / a.Tc, tl = frame % a.Tc, t = a.t0 + tl;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), g = l >> 4, n = l & 15;
  const int S = a.S, T = a.T;
  const size_t fo = ((size_t)bh * T + t) * S * D;
  const size_t sf = (size_t)bh * a.Fs + a.f0 + tl;   // staging frame of (head, frame)
  const size_t so = sf * D * D;
  const int ntile = (S + 15) / 16;

  if (a.norms && tid == 0) {
    float sq = 0.f;
    for (int j = 0; j < NB; ++j) sq += a.norm_part[sf * NB + j];
    a.norms[(size_t)bh * T + t] = sqrtf(sq);
  }

  {
    // stage M^T in LDS; k index of MFMA step kc on lane group g is key g*(D/4)+kc
    float* mt = (float*)smem;                        // [D][D + 1]
    const float* snap = (const float*)a.snap + so;
    for (int x = tid; x < D * D; x += kReadWaves * 64) mt[(x / D) * (D + 1) + (x % D)] = snap[x];
    __syncthreads();
    const float* q = (const float*)a.q + fo;
    float* o = (float*)a.o + fo;
    for (int tile = w; tile < ntile; tile += kReadWaves) {
      const int tok = tile * 16 + n;
      float B[D / 4];
#pragma unroll
      for (int kc = 0; kc < D / 4; ++kc) {
        const float x = (tok < S) ? q[(size_t)tok * D + g * (D / 4) + kc] : 0.f;
        B[kc] = x > 0.f ? x : 0.f;
      }
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < D / 4; ++kc) acc = mfma_f32(mt[(16 * jb + n) * (D + 1) + g * (D / 4) + kc], B[kc], acc);
        if (tok < S) *(f32x4*)(o + (size_t)tok * D + 16 * jb + 4 * g) = acc;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// bf16 readout.  One workgroup per (head, frame); every wave holds M_t^T as A
// operands and walks 32-token chunks of the frame.  Q chunks are read with
// fully coalesced 16-byte loads (a chunk is 32*D contiguous bf16), kept
// RING chunks ahead in registers, passed through ReLU and staged in the
// wave's LDS tile, from which the B operands (token n, 8 consecutive keys) are
// read.  The O chunk is assembled in a second LDS tile and written back with
// the same coalesced pattern.  Out-of-range lanes use an offset beyond the
// buffer: their loads read zeros and their stores are dropped, so the loop is
// branch-free and its wait counts are exact.
// ----------------------------------------------------------------------------
template <int D>
struct ReadShape {
  static constexpr int NB = D / 16, NKC = (D + 31) / 32;
  // Q chunks in flight per wave: at D = 128 the A operands alone take 128
  // registers and a third chunk would spill
  static constexpr int RING = D >= 128 ? 2 : 3;
  static constexpr int UPR = D / 8;              // 16-byte units per token row
  static constexpr int NLD = D / 16;             // 1 KB loads per 32-token chunk (= 32*UPR/64)
  static constexpr int RS = D + 8;               // LDS row stride (elements)
  static constexpr size_t tile_bytes = (size_t)32 * RS * 2;
  // per wave: a Q tile and an O tile
  static constexpr size_t lds_bytes(int waves) { return (size_t)waves * 2 * tile_bytes; }
};

// RW waves per workgroup split the frame's chunks: kReadWaves, or twice that
// for launches with fewer frames than CUs, which also give each frame
// a.nsplit workgroups (a short streaming chunk: a few frames per head, too
// few workgroups to keep the chip's loads in flight).  The chunks go round
// the frame's RW * nsplit waves.  Every output element is computed the same
// way whatever RW and nsplit are.
template <int D, bool FP8, int RW>
__global__ __launch_bounds__(RW * 64, RW > kReadWaves ? 1 : 2) void gdn_readout_kernel(ReadoutArgs a) {
  using Sh = ReadShape<D>;
  using IO = IoFmt<FP8>;
  using raw = typename IO::raw;
  constexpr int NB = Sh::NB, NKC = Sh::NKC, UPR = Sh::UPR, NLD = Sh::NLD, RS = Sh::RS;
  constexpr int RS8 = D + 8;                       // row stride (bytes) of the e4m3 O tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int nsp = a.nsplit;
  const int frame = blockIdx.x / nsp, sp = blockIdx.x % nsp;   // over BH * Tc, then the frame's shares
  const int bh = frame / a.Tc, tl = frame % a.Tc, t = a.t0 + tl;
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, n = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int RWT = RW * nsp, wt = RW * sp + w;      // the frame's waves; this wave's place among them
  uint16_t* const qs = (uint16_t*)(smem + (size_t)w * 2 * Sh::tile_bytes);
  uint16_t* const os = qs + 32 * RS;
  const int S = a.S, T = a.T;
  const uint32_t head_bytes = (uint32_t)T * (uint32_t)S * D * IO::ebytes;
  const size_t head0 = (size_t)bh * T * S * D * IO::ebytes;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc((const unsigned char*)a.q + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t ors = make_rsrc((unsigned char*)a.o + head0, head_bytes);
  const uint32_t fbyte = (uint32_t)t * (uint32_t)S * D * IO::ebytes;   // frame's first byte in the head
  const int nchunk = (S + 31) / 32;
  const int NC = (nchunk + RWT - 1) / RWT;                   // chunk slots per wave
  const size_t sf = (size_t)bh * a.Fs + a.f0 + tl;           // staging frame of (head, frame)

  if (a.norms && a.norm_part && sp == 0 && tid == 0) {
    float sq = 0.f;
    for (int j = 0; j < NB; ++j) sq += a.norm_part[sf * NB + j];
    a.norms[(size_t)bh * T + t] = sqrtf(sq);
  }

  // byte offset of 8-element unit u of a chunk (tokens past S -> beyond the buffer)
  auto unit_off = [&](int ch, int u) -> uint32_t {
    const int tok = ch * 32 + u / UPR;
    return (ch < nchunk && tok < S) ? fbyte + (uint32_t)(ch * 32 * UPR + u) * IO::unit_bytes : kOOB;
  };
  auto load_chunk = [&](int i, raw (&X)[NLD]) {
    const int ch = wt + RWT * i;
#pragma unroll
    for (int j = 0; j < NLD; ++j) X[j] = IO::load_nt(qrs, i < NC ? unit_off(ch, 64 * j + l) : kOOB);
  };

  // A operands: M_t^T rows (value column 16jb + n); k-step kc holds keys
  // 32kc + 4g..+3 and 32kc + 16 + 4g..+3, i.e. the snapshot blocks (jb, 2kc)
  // and (jb, 2kc + 1) of this lane
  const unsigned char* snap = (const unsigned char*)a.snap + sf * D * D * 2;
  u32x4 A[NB][NKC];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb)
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const u32x2 lo = *(const u32x2*)(snap + ((size_t)(jb * NB + 2 * kc) * 64 + l) * 8);
      const u32x2 hi = (2 * kc + 1 < NB) ? *(const u32x2*)(snap + ((size_t)(jb * NB + 2 * kc + 1) * 64 + l) * 8)
                                         : u32x2{0u, 0u};
      A[jb][kc] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  constexpr int RING = Sh::RING;
  raw X[RING][NLD];
#pragma unroll
  for (int r = 0; r < RING; ++r) load_chunk(r, X[r]);
  // The snapshot loads were issued first: one use of the last of them makes
  // the compiler wait for all of them here, once, instead of inside the loop.
  asm volatile("" ::"v"(A[NB - 1][NKC - 1]));
  if (a.norms && !a.norm_part && sp == 0 && w == 0) {
    // state norm from the bf16 snapshot: each element of M_t sits in exactly
    // one lane of one fragment of every wave
    float sq = 0.f;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int e = 0; e < 4; ++e) sq = add_sq_bf16x2(sq, A[jb][kc][e]);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) sq += __shfl_xor(sq, s, 64);
    if (l == 0) a.norms[(size_t)bh * T + t] = sqrtf(sq);
  }

  for (int base = 0; base < NC; base += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int i = base + r;
      const int ch = wt + RWT * i;
      // the loop is unrolled by RING: slots past NC only keep the loads going
      const bool live = i < NC;
      // stage ReLU(Q) of the chunk (row-major, padded rows)
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
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 B[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          // keys in the k-slot order of the A operands
          const uint16_t* rp = qs + (16 * half + n) * RS + 32 * kc + 4 * g;
          const u32x2 lo = *(const u32x2*)rp;
          const u32x2 hi = (32 * kc + 32 <= D) ? *(const u32x2*)(rp + 16) : u32x2{0u, 0u};
          B[kc] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) acc = mfma_bf16(A[jb][kc], B[kc], acc);
          if constexpr (FP8) {
            // one rounding, fp32 -> e4m3
            *(uint32_t*)((unsigned char*)os + (16 * half + n) * RS8 + 16 * jb + 4 * g) = f32x4_to_fp8x4(acc);
          } else {
            const u32x2 pk = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
            *(u32x2*)(os + (16 * half + n) * RS + 16 * jb + 4 * g) = pk;
          }
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int u = 64 * j + l;
        if constexpr (FP8) {
          const u32x2 y = *(const u32x2*)((const unsigned char*)os + (u / UPR) * RS8 + 8 * (u % UPR));
          __builtin_amdgcn_raw_buffer_store_b64(y, ors, i < NC ? unit_off(ch, u) : kOOB, 0, kNT);
        } else {
          const u32x4 y = *(const u32x4*)(os + (u / UPR) * RS + 8 * (u % UPR));
          __builtin_amdgcn_raw_buffer_store_b128(y, ors, i < NC ? unit_off(ch, u) : kOOB, 0, kNT);
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Launchers.
// ----------------------------------------------------------------------------
template <int D, bool BF16>
static hipError_t launch_recurrence_t(const RecurArgs& ra, hipStream_t stream) {
  static DeviceOnce once;
  LaunchInfo li;
  const hipError_t ie = once.get([](int, LaunchInfo&) {
    hipError_t e = hipSuccess;
    if constexpr (BF16) {
      e = hipFuncSetAttribute((const void*)gdn_recur_bf16_kernel<D, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)BfShape<D>::lds_bytes);
      if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)gdn_recur_bf16_kernel<D, false>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)BfShape<D>::lds_bytes);
    } else {
      e = hipFuncSetAttribute((const void*)gdn_recur_f32_kernel<D>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)RecurShapeF32<D>::lds_bytes);
    }
    return e;
  }, &li);
  if (ie != hipSuccess) return ie;
  const int grid = 8 * ((ra.units + 7) / 8);
  if constexpr (BF16) {
    if (ra.beta_mode == 0)
      hipLaunchKernelGGL((gdn_recur_bf16_kernel<D, true>), dim3(grid), dim3(kThreads), BfShape<D>::lds_bytes,
                         stream, ra);
    else
      hipLaunchKernelGGL((gdn_recur_bf16_kernel<D, false>), dim3(grid), dim3(kThreads), BfShape<D>::lds_bytes,
                         stream, ra);
  } else {
    hipLaunchKernelGGL((gdn_recur_f32_kernel<D>), dim3(grid), dim3(kThreads), RecurShapeF32<D>::lds_bytes,
                       stream, ra);
  }
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_readout_t(const ReadoutArgs& ro, hipStream_t stream) {
  constexpr int RW = kReadWaves;
  static DeviceOnce once;
  LaunchInfo li;
  const hipError_t ie = once.get([](int dev, LaunchInfo& info) {
    hipError_t e = hipSuccess;
    if constexpr (BF16) {
      const void* fns[4] = {(const void*)gdn_readout_kernel<D, false, RW>, (const void*)gdn_readout_kernel<D, true, RW>,
                            (const void*)gdn_readout_kernel<D, false, 2 * RW>,
                            (const void*)gdn_readout_kernel<D, true, 2 * RW>};
      const size_t lds[4] = {ReadShape<D>::lds_bytes(RW), ReadShape<D>::lds_bytes(RW),
                             ReadShape<D>::lds_bytes(2 * RW), ReadShape<D>::lds_bytes(2 * RW)};
      for (int i = 0; i < 4 && e == hipSuccess; ++i)
        e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds[i]);
    } else {
      e = hipFuncSetAttribute((const void*)gdn_readout_f32_kernel<D>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, D * (D + 1) * 4);
    }
    if (e == hipSuccess) e = hipDeviceGetAttribute(&info.cus, hipDeviceAttributeMultiprocessorCount, dev);
    return e;
  }, &li);
  if (ie != hipSuccess) return ie;
  const int cus = li.cus;
  const unsigned frames = (unsigned)(ro.BH * ro.Tc);
  ReadoutArgs ra = ro;
  ra.nsplit = 1;
  if constexpr (BF16) {
    // bf16 snapshots: bf16 or e4m3 Q and O; a launch with fewer frames than
    // CUs (a short streaming chunk) takes twice the waves per frame and
    // splits each frame's chunks over up to 2 cus / frames workgroups, at
    // least a chunk per wave
    const bool wide = (int)frames < cus;
    if (wide) {
      const int nchunk = (ro.S + 31) / 32, rw = 2 * RW;
      ra.nsplit = std::max(1, std::min((2 * cus + (int)frames - 1) / (int)frames, (nchunk + rw - 1) / rw));
    }
    const unsigned grid = frames * (unsigned)ra.nsplit;
    const size_t lds = ReadShape<D>::lds_bytes(wide ? 2 * RW : RW);
    const dim3 block(wide ? 2 * RW * 64 : RW * 64);
    if (ra.fp8) {
      if (wide) hipLaunchKernelGGL((gdn_readout_kernel<D, true, 2 * RW>), dim3(grid), block, lds, stream, ra);
      else hipLaunchKernelGGL((gdn_readout_kernel<D, true, RW>), dim3(grid), block, lds, stream, ra);
    } else {
      if (wide) hipLaunchKernelGGL((gdn_readout_kernel<D, false, 2 * RW>), dim3(grid), block, lds, stream, ra);
      else hipLaunchKernelGGL((gdn_readout_kernel<D, false, RW>), dim3(grid), block, lds, stream, ra);
    }
  } else {
    hipLaunchKernelGGL((gdn_readout_f32_kernel<D>), dim3(frames), dim3(kReadWaves * 64),
                       (size_t)D * (D + 1) * 4, stream, ra);
  }
  return hipGetLastError();
}

#define GDN_DISPATCH2(FN, ARGS)                                                                  \
  switch (D) {                                                                                   \
    case 16: return bf16 ? FN<16, true> ARGS : FN<16, false> ARGS;                               \
    case 32: return bf16 ? FN<32, true> ARGS : FN<32, false> ARGS;                               \
    case 48: return bf16 ? FN<48, true> ARGS : FN<48, false> ARGS;                               \
    case 64: return bf16 ? FN<64, true> ARGS : FN<64, false> ARGS;                               \
    case 80: return bf16 ? FN<80, true> ARGS : FN<80, false> ARGS;                               \
    case 96: return bf16 ? FN<96, true> ARGS : FN<96, false> ARGS;                               \
    case 112: return bf16 ? FN<112, true> ARGS : FN<112, false> ARGS;                            \
    case 128: return bf16 ? FN<128, true> ARGS : FN<128, false> ARGS;                            \
    default: return hipErrorInvalidValue;                                                        \
  }

hipError_t launch_recurrence(int D, bool bf16, const RecurArgs& ra, hipStream_t stream) {
  GDN_DISPATCH2(launch_recurrence_t, (ra, stream))
}
hipError_t launch_readout(int D, bool bf16, const ReadoutArgs& ro, hipStream_t stream) {
  GDN_DISPATCH2(launch_readout_t, (ro, stream))
}
#undef GDN_DISPATCH2

}  // namespace gdn
