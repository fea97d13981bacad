// Frame-wise Gated DeltaNet backward on gfx950: the small kernels around the
// adjoint state pass (gdn_gram.hip) and the gradient products (readout
// variants in gdn_kernels.hip).
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
// Z_t = M_{t-1} Lambda_t^T + Lambda_t M_{t-1}^T per (head, frame), written as a
// bf16 block snapshot.  One workgroup of 4 waves per (head, frame): both
// snapshots are staged in LDS; block (R, C) of Z is
//   sum_kc MFMA(rows(M, R, kc), rows(L, C, kc)) + MFMA(rows(L, R, kc), rows(M, C, kc))
// where rows(X, b, kc) gives lane (i, g) the row 16 b + i of X at columns
// 32 kc + 4 g .. + 3 and 32 kc + 16 + 4 g .. + 3 (the k-slot order of the
// state pass), read from the block snapshot with a transposed LDS read: in
// block [jt][I] the 8 bytes at (16 (x / 4) + y) * 8 hold rows 4 (x / 4) ..
// + 3 of column y, and ds_read_b64_tr_b16 with lane j of each 16-lane group
// supplying unit (16 (j % 4) + 4 g + j / 4) hands lane n the row n, columns
// 4 g .. 4 g + 3.  The accumulator of block (R, C) holds, in lane (n, g),
// Z[16 R + 4 g + r][16 C + n]: exactly block [C][R] of the snapshot layout.
// ----------------------------------------------------------------------------
constexpr int kZWaves = 4;

template <int D>
__global__ __launch_bounds__(kZWaves * 64) void gdn_zmat_kernel(ZmatArgs a) {
  constexpr int NB = D / 16, NKC = (NB + 1) / 2;
  constexpr size_t SB = (size_t)D * D * 2;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int fh = blockIdx.x;                       // over BH * T
  const int bh = fh / a.T, t = fh % a.T;
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, n = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  unsigned char* ms = smem;
  unsigned char* ls = smem + SB;
  const __amdgpu_buffer_rsrc_t mrs =
      make_rsrc((const unsigned char*)a.msnap + ((size_t)bh * (a.T + 1) + t) * SB, (uint32_t)SB);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc((const unsigned char*)a.lsnap + ((size_t)bh * a.T + t) * SB,
                                               (uint32_t)SB);
  for (int u = tid; u < (int)(SB / 16); u += kZWaves * 64) {
    *(u32x4*)(ms + (size_t)u * 16) = buf_load16(mrs, (uint32_t)u * 16u);
    *(u32x4*)(ls + (size_t)u * 16) = buf_load16(lrs, (uint32_t)u * 16u);
  }
  __syncthreads();
  const uint32_t trofs = (uint32_t)(((n & 3) * 16 + 4 * g + (n >> 2)) * 8);
  auto rows = [&](const unsigned char* x, int b, int kc) -> u32x4 {
    const u32x2 lo = lds_tr16((const uint16_t*)(x + (size_t)((2 * kc) * NB + b) * 512 + trofs));
    const u32x2 hi = (2 * kc + 1 < NB) ? lds_tr16((const uint16_t*)(x + (size_t)((2 * kc + 1) * NB + b) * 512 + trofs))
                                       : u32x2{0u, 0u};
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  unsigned char* zout = (unsigned char*)a.zsnap + ((size_t)bh * a.T + t) * SB;
  for (int blk = w; blk < NB * NB; blk += kZWaves) {
    const int R = blk / NB, C = blk % NB;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      acc = mfma_bf16(rows(ms, R, kc), rows(ls, C, kc), acc);
      acc = mfma_bf16(rows(ls, R, kc), rows(ms, C, kc), acc);
    }
    const u32x2 pk = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
    *(u32x2*)(zout + ((size_t)(C * NB + R) * 64 + l) * 8) = pk;
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

template <int D>
static hipError_t launch_zmat_t(const ZmatArgs& za, hipStream_t stream) {
  static bool attr_set = false;
  const size_t lds = (size_t)2 * D * D * 2;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gdn_zmat_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((gdn_zmat_kernel<D>), dim3((unsigned)(za.BH * za.T)), dim3(kZWaves * 64), lds, stream, za);
  return hipGetLastError();
}

hipError_t launch_zmat(int D, const ZmatArgs& za, hipStream_t stream) {
  switch (D) {
    case 16: return launch_zmat_t<16>(za, stream);
    case 32: return launch_zmat_t<32>(za, stream);
    case 48: return launch_zmat_t<48>(za, stream);
    case 64: return launch_zmat_t<64>(za, stream);
    case 80: return launch_zmat_t<80>(za, stream);
    case 96: return launch_zmat_t<96>(za, stream);
    case 112: return launch_zmat_t<112>(za, stream);
    case 128: return launch_zmat_t<128>(za, stream);
    default: return hipErrorInvalidValue;
  }
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
