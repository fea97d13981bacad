// Block-causal temporal convolution with a carried-token cache on gfx950.
//
// The causal FFN of the talk "SANA-Video: Efficient Video Generation with
// Block Linear Diffusion Transformer" (its closing part, on temporal
// convolution): a three-tap depthwise convolution along the frame axis, run
// separately at every spatial token and channel.  Blocks of `chunk` frames
// (counted from the call's first frame) see their own next frame, but the
// last frame of a block sees zero in its place (the zero token between
// blocks); every frame sees its previous frame, and the call's first frame
// sees the carried token of the previous call (the cache), or zero:
//
//   y[t] = w[0] left_t + w[1] x[t] + w[2] right_t + bias      (fp32, fma in this order:
//                                                               bias, left, current, right)
//
// The pass is a pure stream (4 bytes per bf16 element, read and write), so it
// is laid out for HBM, not for the matrix cores: a lane owns 16 bytes of
// channels (8 bf16 or 4 fp32) of one spatial token and walks a segment of
// frames, holding the previous and current frame in registers; loads for a
// group of frames are issued together, ahead of their use.  Consecutive lanes
// own consecutive channel groups, so every frame of a wave is one contiguous
// 1 KiB read and write.  A segment re-reads one frame (its left neighbour),
// so segments of kSegFrames frames cost 1/kSegFrames extra reads and give the
// GPU enough waves when B*S*C is small.
//
// The cache: segment 0 of a column reads cache_in first and writes
// cache_out = x[T-1] last, so cache_out may equal cache_in exactly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kTconvThreads = 256;
constexpr int kTconvGroup = 8;     // frames whose loads are issued together
constexpr int kSegFrames = 64;     // frames per segment (a multiple of kTconvGroup)

template <bool F32>
struct TconvIo;
template <>
struct TconvIo<false> {            // bf16: 8 channels per lane
  static constexpr int V = 8;
  __device__ static __forceinline__ void unpack(u32x4 r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo_f32(r[i]);
      f[2 * i + 1] = bf16_hi_f32(r[i]);
    }
  }
  __device__ static __forceinline__ u32x4 pack(const float* f) {
    return u32x4{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
  }
};
template <>
struct TconvIo<true> {             // fp32: 4 channels per lane
  static constexpr int V = 4;
  // whole-vector casts: a bit cast of one element of a vector lvalue (r[i])
  // reads element 0 whatever i is in this compiler
  __device__ static __forceinline__ void unpack(u32x4 r, float* f) {
    const f32x4 v = __builtin_bit_cast(f32x4, r);
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = v[i];
  }
  __device__ static __forceinline__ u32x4 pack(const float* f) {
    return __builtin_bit_cast(u32x4, f32x4{f[0], f[1], f[2], f[3]});
  }
};

__device__ __forceinline__ u32x4 load_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_nt(u32x4 v, u32x4* p) { __builtin_nontemporal_store(v, p); }

// grid: x = column blocks of kTconvThreads lanes (one 16-byte column each),
// y = frame segments, z = batch.
template <bool F32>
__global__ __launch_bounds__(kTconvThreads) void gdn_tconv_kernel(TconvArgs a) {
  using IO = TconvIo<F32>;
  constexpr int V = IO::V;
  const long long cols = a.cols;                       // 16-byte columns per frame: S*C/V
  const long long col = (long long)blockIdx.x * kTconvThreads + threadIdx.x;
  if (col >= cols) return;
  const int b = blockIdx.z, seg = blockIdx.y, T = a.T, chunk = a.chunk;
  const int f0 = seg * a.seg_frames;
  const int f1 = min(T, f0 + a.seg_frames);
  const u32x4* x = (const u32x4*)a.x + (long long)b * T * cols + col;
  u32x4* y = (u32x4*)a.y + (long long)b * T * cols + col;
  const int c0 = (int)(col % a.cols_per_token) * V;    // first channel of this lane

  float wl[V], wc[V], wr[V], bs[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    wl[i] = a.w[c0 + i];
    wc[i] = a.w[a.C + c0 + i];
    wr[i] = a.w[2 * a.C + c0 + i];
    bs[i] = a.bias ? a.bias[c0 + i] : 0.f;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 prev;
  if (f0 > 0)
    prev = load_nt(x + (long long)(f0 - 1) * cols);
  else
    prev = a.cache_in ? *((const u32x4*)a.cache_in + (long long)b * cols + col) : zero;
  u32x4 cur = load_nt(x + (long long)f0 * cols);

  for (int g = f0; g < f1; g += kTconvGroup) {
    u32x4 nx[kTconvGroup];
#pragma unroll
    for (int j = 0; j < kTconvGroup; ++j) {
      const int f = g + 1 + j;                          // right neighbour of frame g + j
      nx[j] = (f < T && f <= f1) ? load_nt(x + (long long)f * cols) : zero;
    }
#pragma unroll
    for (int j = 0; j < kTconvGroup; ++j) {
      const int f = g + j;
      if (f >= f1) break;
      const bool in_block = (f + 1 < T) && ((f + 1) % chunk != 0);
      float l[V], c[V], r[V], o[V];
      IO::unpack(prev, l);
      IO::unpack(cur, c);
      IO::unpack(in_block ? nx[j] : zero, r);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        float acc = bs[i];
        acc = __builtin_fmaf(wl[i], l[i], acc);
        acc = __builtin_fmaf(wc[i], c[i], acc);
        acc = __builtin_fmaf(wr[i], r[i], acc);
        o[i] = acc;
      }
      store_nt(IO::pack(o), y + (long long)f * cols);
      prev = cur;
      cur = nx[j];
    }
  }
  if (seg == 0 && a.cache_out) {
    // x[T-1]: this segment's last frame when it covers the whole call
    const u32x4 last = (f1 == T) ? prev : load_nt(x + (long long)(T - 1) * cols);
    *((u32x4*)a.cache_out + (long long)b * cols + col) = last;
  }
}

}  // namespace

hipError_t launch_tconv(const TconvArgs& in, hipStream_t stream) {
  TconvArgs a = in;
  const int V = a.f32 ? 4 : 8;
  a.cols_per_token = a.C / V;
  a.cols = (long long)a.S * a.cols_per_token;
  a.seg_frames = kSegFrames;
  const long long gx = (a.cols + kTconvThreads - 1) / kTconvThreads;
  const int nseg = (a.T + kSegFrames - 1) / kSegFrames;
  if (gx > 0x7fffffffLL || nseg > 65535 || a.B > 65535) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)gx, (unsigned)nseg, (unsigned)a.B);
  if (a.f32)
    hipLaunchKernelGGL(gdn_tconv_kernel<true>, grid, dim3(kTconvThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(gdn_tconv_kernel<false>, grid, dim3(kTconvThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
