// Device helpers shared by the gfx950 kernels of the frame-wise GDN path:
// vector types, MFMA wrappers, bf16 packing, ReLU on packed bf16, LDS
// transposed reads, buffer resources with out-of-range offsets and an
// LDS-only workgroup barrier.
//
// MFMA lane layouts used (gfx950, wave64; l = lane, g = l/16):
//   v_mfma_f32_16x16x32_bf16: A lane holds row l%16, k = 8g..8g+7;
//                             B lane holds col l%16, k = 8g..8g+7;
//                             C lane holds col l%16, rows 4g..4g+3.
//   v_mfma_f32_16x16x4_f32:   A row l%16, k = g; B col l%16, k = g; C as above.
//   ds_read_b64_tr_b16: in each 16-lane group, lane j supplies the address of
//   4 consecutive 16-bit values (row j/4, columns 4(j%4)..+3 of a 4 x 16 block);
//   lane i receives column i (rows 0..3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

template <int V>
struct Int {
  static constexpr int value = V;
};
// f(Int<0>{}), ..., f(Int<N-1>{}): compile-time loop (every index a constant)
template <int N, int K = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (K < N) {
    f(Int<K>{});
    static_for<N, K + 1>(f);
  }
}

// ReLU on two packed bf16: a negative bf16 has its sign bit set, i.e. it is a
// negative int16, so an int16 max with 0 zeroes it and keeps the rest.
__device__ __forceinline__ uint32_t relu2(uint32_t x) {
  i16x2 v = __builtin_bit_cast(i16x2, x);
  i16x2 z = {0, 0};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(v, z));
}
__device__ __forceinline__ u32x4 relu8(u32x4 x) {
  return u32x4{relu2(x[0]), relu2(x[1]), relu2(x[2]), relu2(x[3])};
}
__device__ __forceinline__ float bf16_lo_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// e4m3 x e4m3 -> fp32, 16x16x32.  Operand lane layout (checked on the GPU
// against a host product of small exact values): lane l holds row (column
// for B) l % 16, k = 8 (l / 16) + j in its byte j; the result as for bf16:
// lane l holds rows 4 (l / 16) + r, column l % 16.  Numerics (measured on
// random finite codes, subnormals included, against exact sums): every
// product is exact, subnormal codes are honoured, but the 32-term sum is not
// fp32-exact: |result - exact| stayed within 2.2e-4 of the sum of |products|.
__device__ __forceinline__ f32x4 mfma_fp8(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b), c, 0,
                                                     0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 8-byte transposed LDS read (see header comment for the lane mapping).
__device__ __forceinline__ u32x2 lds_tr16(const uint16_t* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Transposing 8-byte LDS read of 8-bit elements.  Within each 16-lane group
// the lanes' addresses name 16 rows of 8 bytes, D[i][c] (row i from lane i
// of the group); lane l of the group receives D[l / 8 + 2k][l % 8] in byte k
// (checked on the GPU with a pattern of known bytes).
__device__ __forceinline__ u32x2 lds_tr8(const unsigned char* p) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
  return __builtin_bit_cast(u32x2, r);
}
// ReLU of 8 OCP E4M3 codes: a code with the sign bit set (negative values,
// -0 and the negative NaN) becomes +0, as the bf16 ReLU of its exact value.
__device__ __forceinline__ u32x2 relu_e4m3x8(u32x2 x) {
  const uint32_t s0 = (x[0] >> 7) & 0x01010101u, s1 = (x[1] >> 7) & 0x01010101u;
  return u32x2{x[0] & ~(s0 * 0xFFu), x[1] & ~(s1 * 0xFFu)};
}

// Wave-local LDS ordering: LDS operations of one wave complete in order; the
// fence stops the compiler from moving LDS accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One state update of the Gram form, gm*m - bg*p + w, as two fused
// multiply-adds in a fixed order, so that every kernel running it (the state
// pass and the one-launch forward) rounds the same way.
__device__ __forceinline__ float state_update(float gm, float m, float bg, float p, float w) {
  return __builtin_fmaf(gm, m, __builtin_fmaf(-bg, p, w));
}
// Adds the squares of the two bf16 of a packed word to sq, in a fixed order.
__device__ __forceinline__ float add_sq_bf16x2(float sq, uint32_t w) {
  const float x = __builtin_bit_cast(float, w << 16), y = __builtin_bit_cast(float, w & 0xffff0000u);
  return __builtin_fmaf(y, y, __builtin_fmaf(x, x, sq));
}

// Pack two floats into two bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// OCP e4m3 (the "fn" variant: exponent bias 7, no infinities, 0x7F and 0xFF
// are NaN).  v_cvt_pk_f32_fp8 decodes two bytes exactly, and every e4m3 value
// is also exact in bf16, so eight bytes become eight bf16 with no rounding.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 x) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[0], false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[0], true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[1], false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[1], true);
  return u32x4{pack_bf16(a[0], a[1]), pack_bf16(b[0], b[1]), pack_bf16(c[0], c[1]), pack_bf16(d[0], d[1])};
}
// Four floats to four e4m3 bytes, in order: round to nearest even, and a
// magnitude past the rounding range of the largest finite value (448)
// becomes NaN (v_cvt_pk_fp8_f32).
__device__ __forceinline__ uint32_t f32x4_to_fp8x4(f32x4 v) {
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], p, true);
  return (uint32_t)p;
}

// XCD-aware unit for this workgroup: units are split into 8 contiguous ranges,
// range x is served by the workgroups that land on XCD x (ids = x mod 8).
__device__ __forceinline__ int xcd_unit(int units) {
  const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int start = (int)(((long long)x * units) >> 3);
  const int end = (int)(((long long)(x + 1) * units) >> 3);
  return (start + slot < end) ? start + slot : -1;
}

constexpr uint32_t kOOB = 0x80000000u;      // offset past every buffer (buffers are < 2 GiB)
constexpr int kBufWord3 = 0x00020000;       // gfx9 buffer descriptor word 3 (raw 32-bit dwords)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}
// Cache-policy bits of a buffer instruction: kNT marks data that is touched
// once (Q, K, V, O, the per-frame B_t tiles) as streaming.  Under heavy read
// traffic it measurably lowers the cost of the passes' own stores, which
// otherwise compete with the streamed lines for L2 residency.
constexpr int kNT = 2;
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT));
}
// Element format of Q, K, V and O.  The kernels stage every operand as bf16
// in LDS; they load a tensor in units of 8 elements per lane -- 16 bytes of
// bf16 or 8 bytes of e4m3 -- and convert the unit on its way to LDS.
template <bool FP8>
struct IoFmt;
template <>
struct IoFmt<false> {
  static constexpr uint32_t ebytes = 2;
  static constexpr uint32_t unit_bytes = 16;
  using raw = u32x4;
  __device__ static __forceinline__ raw load_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) { return buf_load16_nt(r, off); }
  __device__ static __forceinline__ u32x4 to_bf16(raw x) { return x; }
};
template <>
struct IoFmt<true> {
  static constexpr uint32_t ebytes = 1;
  static constexpr uint32_t unit_bytes = 8;
  using raw = u32x2;
  __device__ static __forceinline__ raw load_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNT));
  }
  __device__ static __forceinline__ u32x4 to_bf16(raw x) { return fp8x8_to_bf16x8(x); }
};

// LDS-only workgroup barrier: waits for this wave's LDS operations, not for
// its outstanding global loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace gdn
