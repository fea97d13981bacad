// Frame-wise Gated DeltaNet backward on gfx950: the initial-state snapshot,
// the fused dV/dK pass (which forms Z_t itself) and the dgamma/dbeta
// reduction.  The forward
// replay, the fused C_t/dQ pass and the adjoint state pass live in
// gdn_gram.hip beside the forward passes they mirror.
//
// The gradients are those of the forward described in the SANA-WM news
// article ("NVIDIA Apresenta SANA-WM ...", section "1. Atencao Linear Hibrida
// com Gated DeltaNet (GDN)").  With Lambda_t = dL/dM_t from the adjoint pass,
// per frame t (Kf = c ReLU(K_t), w_t = 1 ERASE or beta_t WRITE):
//   dQ_t = (dO_t M_t^T) * [Q_t > 0]
//   dV_t = w_t Kf_t Lambda_t
//   dK_t = (c w_t V_t Lambda_t^T - c^2 b_t g_t ReLU(K_t) Z_t) * [K_t > 0],
//          Z_t = M_{t-1} Lambda_t^T + Lambda_t M_{t-1}^T
// and dg_t, db_t from the adjoint pass's partial sums.
//
// Snapshot block layout (as the forward's): a D x D matrix X is stored as
// (D/16)^2 blocks of 512 bytes, block [jt][I] at ((jt * NB + I) * 512), in
// which lane l = 16 g + n holds X[16 I + 4 g + r][16 jt + n], r = 0..3, at
// bytes 8 l .. 8 l + 7.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// ----------------------------------------------------------------------------
// bf16 block snapshot of an fp32 state [BH][D][D] (zeros when state is null),
// one thread per element.
// ----------------------------------------------------------------------------
__global__ void gdn_state_snapshot_kernel(const float* state, uint16_t* snap, int BH, int D,
                                          long long slot_stride_bytes) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long per = (long long)D * D;
  if (idx >= (long long)BH * per) return;
  const int bh = (int)(idx / per), e = (int)(idx % per);
  const int row = e / D, col = e % D, NB = D / 16;
  const int I = row >> 4, g = (row & 15) >> 2, r = row & 3, jt = col >> 4, n = col & 15;
  const float x = state ? state[idx] : 0.f;
  unsigned char* base = (unsigned char*)snap + (size_t)bh * slot_stride_bytes;
  const size_t off = ((size_t)(jt * NB + I) * 64 + (16 * g + n)) * 8 + 2 * r;
  const __bf16 b = (__bf16)x;
  *(uint16_t*)(base + off) = __builtin_bit_cast(uint16_t, b);
}

// ----------------------------------------------------------------------------
// dV_t and dK_t in one pass over K_t and V_t.  One workgroup of 4 waves per
// (head, frame).  The frame's 32-token chunks of K and V are loaded once,
// cooperatively (1 KB pieces spread over the waves, kDvkRing chunks ahead in
// registers), and staged in a double-buffered LDS tile, K through ReLU.  Wave
// w owns the output column blocks jb = w, w + 4 (< D/16) of both gradients and
// holds, for them, the MFMA A operands of Lambda_t, of Lambda_t^T and of
// Z_t = M_{t-1} Lambda_t^T + Lambda_t M_{t-1}^T (the readout's operand
// layout).  Lambda_t^T and Z_t come from the Lambda_t and M_{t-1} snapshots
// staged in LDS before the token loop: transposed LDS reads for the row
// operands and two MFMA chains per Z block, whose output layout is already
// the operand layout.  Per chunk and 16-token half it forms
//   dV = c w ReLU(K) Lambda,   dK = (c w V Lambda^T - c^2 b g ReLU(K) Z) * [K > 0]
// (the mask read from the staged ReLU(K)), assembles both in LDS tiles and
// stores them with the same coalesced 1 KB pieces.
// ----------------------------------------------------------------------------
constexpr int kDvkWaves = 4;
constexpr int kDvkRing = 4;

template <int D>
struct DvkShape {
  static constexpr int NB = D / 16, NKC = (NB + 1) / 2;
  static constexpr int UPR = D / 8;                                   // 16-byte units per token row
  static constexpr int NLD = D / 16;                                  // 1 KB pieces per chunk of one tensor
  static constexpr int LPW = (2 * NLD + kDvkWaves - 1) / kDvkWaves;   // pieces per wave per chunk
  static constexpr int JPW = (NB + kDvkWaves - 1) / kDvkWaves;        // column blocks per wave
  static constexpr int RS = D + 8;                                    // LDS row stride (elements)
  static constexpr size_t tile_bytes = (size_t)32 * RS * 2;
  // K, V x 2 buffers and the dV, dK tiles; before the token loop the same
  // space holds the Lambda_t and M_{t-1} snapshots
  static constexpr size_t snap_bytes = (size_t)D * D * 2;
  static constexpr size_t lds_bytes = 6 * tile_bytes > 2 * snap_bytes ? 6 * tile_bytes : 2 * snap_bytes;
};

template <int D, bool WRITE>
__global__ __launch_bounds__(kDvkWaves * 64, 2) void gdn_dvdk_kernel(DvkArgs a) {
  using Sh = DvkShape<D>;
  constexpr int NB = Sh::NB, NKC = Sh::NKC, UPR = Sh::UPR, NLD = Sh::NLD, LPW = Sh::LPW, JPW = Sh::JPW;
  constexpr int RS = Sh::RS;
  static_assert(2 * Sh::snap_bytes <= Sh::lds_bytes, "the Lambda and M snapshots are staged in the tiles' space");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int T = a.T, S = a.S;
  const int fh = blockIdx.x, bh = fh / a.Tc, t = a.t0 + fh % a.Tc;
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, n = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t head_bytes = (uint32_t)T * (uint32_t)S * D * 2u;
  const size_t head0 = (size_t)bh * T * S * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc((const unsigned char*)a.k + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const unsigned char*)a.v + head0, head_bytes);
  const __amdgpu_buffer_rsrc_t dvrs = make_rsrc(a.dv ? (unsigned char*)a.dv + head0 : nullptr, a.dv ? head_bytes : 0u);
  const __amdgpu_buffer_rsrc_t dkrs = make_rsrc(a.dk ? (unsigned char*)a.dk + head0 : nullptr, a.dk ? head_bytes : 0u);
  const uint32_t fbyte = (uint32_t)t * (uint32_t)S * D * 2u;
  const float bt = a.beta[(size_t)bh * T + t], gm = a.gamma[(size_t)bh * T + t];
  const float cw = a.kscale * (WRITE ? bt : 1.f), cz = -a.kscale * a.kscale * bt * gm;

  // weights of this wave's column blocks: Lambda_t and Lambda_t^T from the
  // Lambda snapshot, Z_t = M_{t-1} Lambda_t^T + Lambda_t M_{t-1}^T computed
  // here from both snapshots staged in LDS
  const size_t snb = ((size_t)bh * T + t) * D * D * 2;
  const unsigned char* lsn = (const unsigned char*)a.lsnap + snb;
  const unsigned char* msn = (const unsigned char*)a.msnap + ((size_t)bh * (T + 1) + t) * D * D * 2;
  unsigned char* const ls = smem;                                  // Lambda_t
  unsigned char* const ms = smem + Sh::snap_bytes;                 // M_{t-1}
  for (int u = tid; u < D * D * 2 / 16; u += kDvkWaves * 64) {
    *(u32x4*)(ls + (size_t)u * 16) = *(const u32x4*)(lsn + (size_t)u * 16);
    *(u32x4*)(ms + (size_t)u * 16) = *(const u32x4*)(msn + (size_t)u * 16);
  }
  __syncthreads();
  const uint32_t trofs = (uint32_t)(((n & 3) * 16 + 4 * g + (n >> 2)) * 8);
  // rows 16 b .. 16 b + 15 of a staged snapshot X as an MFMA operand over the
  // 32-wide k-step kc (lane n: row 16 b + n, columns 32 kc + 8 g' ..)
  auto rows = [&](const unsigned char* x, int b, int kc) -> u32x4 {
    const u32x2 lo = lds_tr16((const uint16_t*)(x + (size_t)((2 * kc) * NB + b) * 512 + trofs));
    const u32x2 hi = (2 * kc + 1 < NB) ? lds_tr16((const uint16_t*)(x + (size_t)((2 * kc + 1) * NB + b) * 512 + trofs))
                                       : u32x2{0u, 0u};
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  u32x4 AL[JPW][NKC], AT[JPW][NKC], AZ[JPW][NKC];
#pragma unroll
  for (int i = 0; i < JPW; ++i) {
    const int jb = w + kDvkWaves * i;
    const bool has = jb < NB;
    const int jj = has ? jb : 0;
    u32x4 MT[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const bool h2 = 2 * kc + 1 < NB;
      const size_t b0 = (size_t)(jj * NB + 2 * kc) * 512 + l * 8, b1 = b0 + 512;
      const u32x2 llo = *(const u32x2*)(lsn + b0), lhi = h2 ? *(const u32x2*)(lsn + b1) : u32x2{0u, 0u};
      AL[i][kc] = u32x4{llo[0], llo[1], lhi[0], lhi[1]};
      AT[i][kc] = rows(ls, jj, kc);          // Lambda rows of block jb = Lambda^T columns
      MT[kc] = rows(ms, jj, kc);
    }
    // Z block (R, jb) in the MFMA output layout is the snapshot block layout
    // that AZ takes: lane (n, g) holds Z[16 R + 4 g + r][16 jb + n]
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      u32x2 half[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int R = 2 * kc + hh;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (R < NB) {
#pragma unroll
          for (int k2 = 0; k2 < NKC; ++k2) {
            acc = mfma_bf16(rows(ms, R, k2), AT[i][k2], acc);
            acc = mfma_bf16(rows(ls, R, k2), MT[k2], acc);
          }
        }
        half[hh] = u32x2{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
      }
      AZ[i][kc] = u32x4{half[0][0], half[0][1], half[1][0], half[1][1]};
    }
  }
  __syncthreads();

  uint16_t* const ovt = (uint16_t*)(smem + 4 * Sh::tile_bytes);    // dV tile
  uint16_t* const okt = ovt + 32 * RS;                              // dK tile
  const int nch = (S + 31) / 32;
  auto unit_off = [&](int ch, int u) -> uint32_t {
    const int tok = ch * 32 + u / UPR;
    return (ch < nch && tok < S) ? fbyte + (uint32_t)(ch * 32 * UPR + u) * 16u : kOOB;
  };
  // piece p of a chunk: p < NLD keys, NLD <= p < 2 NLD values (and, when
  // storing, dV then dK); lane l carries 16-byte unit 64 (p mod NLD) + l
  auto load_chunk = [&](int ch, u32x4 (&X)[LPW]) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int p = w + kDvkWaves * i;
      const uint32_t off = p < 2 * NLD ? unit_off(ch, 64 * (p % NLD) + l) : kOOB;
      X[i] = buf_load16_nt(p < NLD ? krs : vrs, off);
    }
  };
  auto stage = [&](int buf, const u32x4 (&X)[LPW]) {
    uint16_t* kt = (uint16_t*)(smem + (size_t)buf * 2 * Sh::tile_bytes);
    uint16_t* vt = kt + 32 * RS;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int p = w + kDvkWaves * i;
      if (p < 2 * NLD) {
        const int u = 64 * (p % NLD) + l;
        *(u32x4*)((p < NLD ? kt : vt) + (u / UPR) * RS + 8 * (u % UPR)) = p < NLD ? relu8(X[i]) : X[i];
      }
    }
  };

  u32x4 X[kDvkRing][LPW];
#pragma unroll
  for (int r = 0; r < kDvkRing; ++r) load_chunk(r, X[r]);
  const int nit = (nch + kDvkRing - 1) / kDvkRing * kDvkRing;
  for (int base = 0; base < nit; base += kDvkRing) {
#pragma unroll
    for (int r = 0; r < kDvkRing; ++r) {
      const int c = base + r;
      stage(r & 1, X[r]);
      load_chunk(c + kDvkRing, X[r]);
      lds_barrier();
      if (c < nch) {
        const uint16_t* kt = (const uint16_t*)(smem + (size_t)(r & 1) * 2 * Sh::tile_bytes);
        const uint16_t* vt = kt + 32 * RS;
#pragma unroll
        for (int i = 0; i < JPW; ++i) {
          const int jb = w + kDvkWaves * i;
          if (jb < NB) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              u32x4 BK[NKC], BV[NKC];
#pragma unroll
              for (int kc = 0; kc < NKC; ++kc) {
                const int ro = (16 * half + n) * RS + 32 * kc + 4 * g;
                const bool h2 = 32 * kc + 32 <= D;
                const u32x2 klo = *(const u32x2*)(kt + ro), khi = h2 ? *(const u32x2*)(kt + ro + 16) : u32x2{0u, 0u};
                const u32x2 vlo = *(const u32x2*)(vt + ro), vhi = h2 ? *(const u32x2*)(vt + ro + 16) : u32x2{0u, 0u};
                BK[kc] = u32x4{klo[0], klo[1], khi[0], khi[1]};
                BV[kc] = u32x4{vlo[0], vlo[1], vhi[0], vhi[1]};
              }
              f32x4 av = {0.f, 0.f, 0.f, 0.f}, a1 = av, a2 = av;
#pragma unroll
              for (int kc = 0; kc < NKC; ++kc) {
                av = mfma_bf16(AL[i][kc], BK[kc], av);
                a1 = mfma_bf16(AT[i][kc], BV[kc], a1);
                a2 = mfma_bf16(AZ[i][kc], BK[kc], a2);
              }
              const int oo = (16 * half + n) * RS + 16 * jb + 4 * g;
              const u32x2 kr = *(const u32x2*)(kt + oo);     // ReLU(K) at the same (token, column)
              f32x4 dk;
#pragma unroll
              for (int e = 0; e < 4; ++e) dk[e] = cw * a1[e] + cz * a2[e];
              dk[0] = (kr[0] & 0xffffu) ? dk[0] : 0.f;
              dk[1] = (kr[0] >> 16) ? dk[1] : 0.f;
              dk[2] = (kr[1] & 0xffffu) ? dk[2] : 0.f;
              dk[3] = (kr[1] >> 16) ? dk[3] : 0.f;
              *(u32x2*)(ovt + oo) = u32x2{pack_bf16(cw * av[0], cw * av[1]), pack_bf16(cw * av[2], cw * av[3])};
              *(u32x2*)(okt + oo) = u32x2{pack_bf16(dk[0], dk[1]), pack_bf16(dk[2], dk[3])};
            }
          }
        }
      }
      lds_barrier();
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int p = w + kDvkWaves * i;
        if (p < 2 * NLD) {
          const int u = 64 * (p % NLD) + l;
          const u32x4 y = *(const u32x4*)((p < NLD ? ovt : okt) + (u / UPR) * RS + 8 * (u % UPR));
          __builtin_amdgcn_raw_buffer_store_b128(y, p < NLD ? dvrs : dkrs, unit_off(c, u), 0, kNT);
        }
      }
    }
  }
}

template <int D>
static hipError_t launch_dvdk_t(const DvkArgs& da, hipStream_t stream) {
  static DeviceOnce once;
  LaunchInfo li;
  const hipError_t ie = once.get([](int, LaunchInfo&) {
    hipError_t e = hipFuncSetAttribute((const void*)gdn_dvdk_kernel<D, false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)DvkShape<D>::lds_bytes);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)gdn_dvdk_kernel<D, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)DvkShape<D>::lds_bytes);
    return e;
  }, &li);
  if (ie != hipSuccess) return ie;
  const dim3 grid((unsigned)(da.BH * da.Tc)), block(kDvkWaves * 64);
  if (da.beta_mode == 0)
    hipLaunchKernelGGL((gdn_dvdk_kernel<D, false>), grid, block, DvkShape<D>::lds_bytes, stream, da);
  else
    hipLaunchKernelGGL((gdn_dvdk_kernel<D, true>), grid, block, DvkShape<D>::lds_bytes, stream, da);
  return hipGetLastError();
}

hipError_t launch_dvdk(int D, const DvkArgs& da, hipStream_t stream) {
  switch (D) {
    case 16: return launch_dvdk_t<16>(da, stream);
    case 32: return launch_dvdk_t<32>(da, stream);
    case 48: return launch_dvdk_t<48>(da, stream);
    case 64: return launch_dvdk_t<64>(da, stream);
    case 80: return launch_dvdk_t<80>(da, stream);
    case 96: return launch_dvdk_t<96>(da, stream);
    case 112: return launch_dvdk_t<112>(da, stream);
    case 128: return launch_dvdk_t<128>(da, stream);
    default: return hipErrorInvalidValue;
  }
}

// ----------------------------------------------------------------------------
// dg_t and db_t from the adjoint pass's per-wave partial sums, summed over
// the head's (value tile, block) pairs in a fixed order.
// ----------------------------------------------------------------------------
__global__ void gdn_adjoint_reduce_kernel(const float* part, const float* gamma, const float* beta,
                                          float* dgamma, float* dbeta, int BH, int T, int NB, int write_mode) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;    // (head, frame)
  if (idx >= BH * T) return;
  const float* p = part + (size_t)idx * NB * NB * 4;
  double s1 = 0.0, s2 = 0.0, s3 = 0.0;
  for (int k = 0; k < NB * NB; ++k) {
    s1 += p[4 * k];
    s2 += p[4 * k + 1];
    s3 += p[4 * k + 2];
  }
  const double g = gamma[idx], b = beta[idx];
  if (dgamma) dgamma[idx] = (float)(s1 - b * s2);
  if (dbeta) dbeta[idx] = (float)(-g * s2 + (write_mode ? s3 : 0.0));
}


hipError_t launch_state_snapshot(const float* state, void* snap, int BH, int D, size_t slot_stride_bytes,
                                 hipStream_t stream) {
  const long long total = (long long)BH * D * D;
  const unsigned grid = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(gdn_state_snapshot_kernel, dim3(grid), dim3(256), 0, stream, state, (uint16_t*)snap, BH, D,
                     (long long)slot_stride_bytes);
  return hipGetLastError();
}

hipError_t launch_adjoint_reduce(const float* part, const float* gamma, const float* beta, float* dgamma,
                                 float* dbeta, int BH, int T, int D, int beta_mode, hipStream_t stream) {
  const int total = BH * T;
  hipLaunchKernelGGL(gdn_adjoint_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, part,
                     gamma, beta, dgamma, dbeta, BH, T, D / 16, beta_mode);
  return hipGetLastError();
}

}  // namespace gdn
