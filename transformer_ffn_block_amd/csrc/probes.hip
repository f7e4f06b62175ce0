// HBM bandwidth probes: a read-only stream and a read+write copy.
//
// A read-only ceiling and a read+write ceiling are different references,
// and weight streaming must be priced against the read-only one ("Unfusing
// a Kernel Made It 1.63x Faster", "Two published claims we got wrong").
// Both kernels use 16-byte lane-contiguous accesses in a grid-stride loop
// with four independent loads in flight per lane; the read probe's grid is a
// parameter so callers can sweep occupancy ("Megakernels on Mac",
// "Bandwidth and memory measurements": best of a sweep, not one geometry).
#include <atomic>

#include "common.h"
#include "launch.h"

namespace ffn {

__global__ __launch_bounds__(256) void probe_read(const uint4* __restrict__ src, int64_t n,
                                                  uint4* __restrict__ sink) {
  uint4 acc = make_uint4(0, 0, 0, 0);
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = ld_nt(src + i);
    const uint4 b = ld_nt(src + i + stride);
    const uint4 c = ld_nt(src + i + 2 * stride);
    const uint4 d = ld_nt(src + i + 3 * stride);
    acc.x ^= a.x ^ b.x ^ c.x ^ d.x;
    acc.y ^= a.y ^ b.y ^ c.y ^ d.y;
    acc.z ^= a.z ^ b.z ^ c.z ^ d.z;
    acc.w ^= a.w ^ b.w ^ c.w ^ d.w;
  }
  for (; i < n; i += stride) {
    const uint4 a = src[i];
    acc.x ^= a.x;
    acc.y ^= a.y;
    acc.z ^= a.z;
    acc.w ^= a.w;
  }
  // a data-dependent store the compiler cannot remove, practically never taken
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// Copy with a grid-stride loop (the grid is a parameter: workgroups per CU).
template <bool NT>
__global__ __launch_bounds__(256) void probe_copy_stride(const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = ld_nt(src + i), b = ld_nt(src + i + stride), c = ld_nt(src + i + 2 * stride),
                d = ld_nt(src + i + 3 * stride);
    st16<NT>(dst + i, a);
    st16<NT>(dst + i + stride, b);
    st16<NT>(dst + i + 2 * stride, c);
    st16<NT>(dst + i + 3 * stride, d);
  }
  for (; i < n; i += stride) st16<NT>(dst + i, ld_nt(src + i));
}

// Copy in contiguous 16 KiB chunks, one workgroup each (the access pattern
// of a row-per-wave elementwise kernel: every workgroup streams its own
// contiguous span, no grid-stride interleaving).
constexpr int64_t kCopyChunk = 256 * 4;  // 16-byte units per workgroup
template <bool NT>
__global__ __launch_bounds__(256) void probe_copy_chunk(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * kCopyChunk + threadIdx.x;
  if (base + 3 * 256 < n) {
    const uint4 a = ld_nt(src + base), b = ld_nt(src + base + 256), c = ld_nt(src + base + 512),
                d = ld_nt(src + base + 768);
    st16<NT>(dst + base, a);
    st16<NT>(dst + base + 256, b);
    st16<NT>(dst + base + 512, c);
    st16<NT>(dst + base + 768, d);
  } else {
    for (int64_t i = base; i < n && i < (int64_t)(blockIdx.x + 1) * kCopyChunk; i += 256)
      st16<NT>(dst + i, ld_nt(src + i));
  }
}

// Dense bf16 matrix-core loop: every wave keeps 8 independent 16x16x32
// accumulations in flight for `iters` rounds (8 MFMAs, 131072 flop per
// round), operands in registers, nothing from memory.  The result is
// stored only if it equals a value it practically never takes, so the
// MFMAs cannot be removed.
__global__ __launch_bounds__(256) void probe_mfma(int iters, float* __restrict__ sink) {
  const unsigned lane = threadIdx.x & 63;
  const uint4 a = make_uint4(0x3F803F80u ^ (lane & 7), 0x3F803F81u, 0xBF80BF80u, 0x3F003F00u ^ lane);
  const uint4 b = make_uint4(0x3E803E80u, 0x3F803F80u ^ (lane >> 3), 0x3F803F80u, 0xBE80BE80u);
  // distinct start values: no two chains compute the same sequence, so none
  // can be merged with another
  f32x4 c0 = {0, 0, 0, 0}, c1 = {1, 1, 1, 1}, c2 = {2, 2, 2, 2}, c3 = {3, 3, 3, 3};
  f32x4 c4 = {4, 4, 4, 4}, c5 = {5, 5, 5, 5}, c6 = {6, 6, 6, 6}, c7 = {7, 7, 7, 7};
  for (int it = 0; it < iters; ++it) {
    c0 = mfma16(a, b, c0);
    c1 = mfma16(b, a, c1);
    c2 = mfma16(a, a, c2);
    c3 = mfma16(b, b, c3);
    c4 = mfma16(a, b, c4);
    c5 = mfma16(b, a, c5);
    c6 = mfma16(a, a, c6);
    c7 = mfma16(b, b, c7);
  }
  const f32x4 t = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  const float v = t[0] + t[1] + t[2] + t[3];
  if (v == 1234.5678f) sink[blockIdx.x * 256 + threadIdx.x] = v;
}

// queried once per device (grid sizes read it on every launch)
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && (cus = cached[dev].load(std::memory_order_relaxed)) > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  if (dev >= 0 && dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int probe_read_groups(int waves_per_cu) {
  const int g = device_cus() * waves_per_cu / 4;
  return g > 0 ? g : 1;
}

hipError_t launch_probe_read(const void* src, size_t bytes, void* sink, int waves_per_cu,
                             hipStream_t s) {
  FFN_DISPATCH(probe_read, dim3((unsigned)probe_read_groups(waves_per_cu)), dim3(256), 0,
                     s, (const uint4*)src, (int64_t)(bytes / 16), (uint4*)sink);
  return hipGetLastError();
}

int probe_copy_groups(size_t bytes, int groups_per_cu) {
  const int64_t n = (int64_t)(bytes / 16);
  int64_t g = groups_per_cu > 0 ? (int64_t)device_cus() * groups_per_cu : (n + kCopyChunk - 1) / kCopyChunk;
  if (groups_per_cu > 0 && g > (n + 255) / 256) g = (n + 255) / 256;
  return (int)(g < 1 ? 1 : g);
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, int groups_per_cu,
                             bool nontemporal, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  const dim3 grid((unsigned)probe_copy_groups(bytes, groups_per_cu));
  const uint4* a = (const uint4*)src;
  uint4* b = (uint4*)dst;
  if (groups_per_cu > 0) {
    if (nontemporal)
      FFN_DISPATCH(probe_copy_stride<true>, grid, dim3(256), 0, s, a, b, n);
    else
      FFN_DISPATCH(probe_copy_stride<false>, grid, dim3(256), 0, s, a, b, n);
  } else {
    if (nontemporal)
      FFN_DISPATCH(probe_copy_chunk<true>, grid, dim3(256), 0, s, a, b, n);
    else
      FFN_DISPATCH(probe_copy_chunk<false>, grid, dim3(256), 0, s, a, b, n);
  }
  return hipGetLastError();
}

int probe_mfma_groups(int waves_per_cu) { return probe_read_groups(waves_per_cu); }

hipError_t launch_probe_mfma(int iters, int waves_per_cu, float* sink, hipStream_t s) {
  FFN_DISPATCH(probe_mfma, dim3((unsigned)probe_mfma_groups(waves_per_cu)), dim3(256), 0, s, iters,
               sink);
  return hipGetLastError();
}

}  // namespace ffn
