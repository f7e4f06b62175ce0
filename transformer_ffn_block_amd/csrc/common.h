// Device-side helpers shared by the gfx950 kernels of libffn.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffn {

typedef uint16_t bf16_t;  // raw bf16 storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) loads: data read once, not worth keeping in cache.
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt(const uint2* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

// 16-byte store; NT = streaming (non-temporal) store
template <bool NT>
__device__ __forceinline__ void st16(uint4* p, const uint4& v) {
  if (NT) {
    u32x4 w;
    w.x = v.x; w.y = v.y; w.z = v.z; w.w = v.w;
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
  } else {
    *p = v;
  }
}

// v if keep else 0, component-wise (a ternary on the struct type would go
// through private memory)
__device__ __forceinline__ uint4 keep_or_zero(bool keep, const uint4& v) {
  const uint32_t m = keep ? 0xFFFFFFFFu : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// Buffer resource over [base, base + bytes) (bytes < 2^31).  A buffer load
// whose offset is past the range returns zeros without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0x7FFFFFFFL ? bytes : 0x7FFFFFFFL),
                                           0x00020000);
}
constexpr unsigned kOutOfRange = 0x80000000u;  // a buffer offset that is never in range

// 16-byte streaming (non-temporal) buffer load at a byte offset
__device__ __forceinline__ uint4 buf_ld_nt(__amdgpu_buffer_rsrc_t r, unsigned off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte cached buffer load at a byte offset
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte buffer load straight into LDS: lane i's 16 bytes land at
// lds + 16*i (lds must be wave-uniform).  AUX 2 = streaming (non-temporal).
template <int AUX>
__device__ __forceinline__ void buf_ld_lds16(__amdgpu_buffer_rsrc_t r, void* lds, unsigned off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           (int)off, 0, 0, AUX);
}

// The same with a wave-uniform byte offset added in the scalar offset
// operand (every byte addressed must lie inside the resource).
template <int AUX>
__device__ __forceinline__ void buf_ld_lds16s(__amdgpu_buffer_rsrc_t r, void* lds, unsigned off,
                                              int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           (int)off, soff, 0, AUX);
}

__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ bf16_t f2bf(float v) {
  return (bf16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
}

// the 8 bf16 of a 16-byte chunk, widened to fp32
__device__ __forceinline__ void unpack8(const uint4& v, float* o) {
  o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xFFFF0000u);
  o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xFFFF0000u);
  o[4] = __uint_as_float(v.z << 16); o[5] = __uint_as_float(v.z & 0xFFFF0000u);
  o[6] = __uint_as_float(v.w << 16); o[7] = __uint_as_float(v.w & 0xFFFF0000u);
}
__device__ __forceinline__ uint4 pack8(const float* o) {
  return make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                    pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
}

// acc + the sum of squares of the 8 bf16 of a 16-byte chunk, straight from
// the packed pairs (v_dot2c_f32_bf16: four instructions instead of eight
// unpacked FMAs; each square is exact in fp32)
__device__ __forceinline__ float sumsq8(const uint4& v, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.x), __builtin_bit_cast(bf16x2, v.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.y), __builtin_bit_cast(bf16x2, v.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.z), __builtin_bit_cast(bf16x2, v.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.w), __builtin_bit_cast(bf16x2, v.w), acc, false);
  return acc;
}

// silu(v) * u in fp32: v * (1 / (1 + e^-v)) * u, the reciprocal from
// v_rcp_f32 (within 1 ulp; the result is rounded to bf16 afterwards) rather
// than an IEEE division, whose correction sequence made the SwiGLU epilogue
// of the fused prefill GEMM ~2% of its time (1.400 -> 1.374 ms).  For
// v -> -inf (finite), e^-v overflows to +inf, its reciprocal is 0 and the
// product is -0, the correct limit.
__device__ __forceinline__ float silu_mul(float v, float u) {
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;
}

// Sum over the 64 lanes of a wavefront (butterfly, every lane gets the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

}  // namespace ffn
