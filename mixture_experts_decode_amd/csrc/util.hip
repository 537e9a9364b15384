// Measurement kernels: contiguous copy (the bandwidth denominator, as in the
// warp-decode post's hardware-efficiency section), read-only streaming, and
// a fill used to evict caches between timed calls.  Also the per-device
// compute-unit count cache.

#include <atomic>

#include "device.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kUtilBlock = 256;

__global__ __launch_bounds__(kUtilBlock) void copy_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, size_t n) {
  size_t i = (size_t)blockIdx.x * kUtilBlock + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kUtilBlock;
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 a = __builtin_nontemporal_load(src + i);
    u32x4 b = __builtin_nontemporal_load(src + i + stride);
    u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(kUtilBlock) void read_kernel(const u32x4* __restrict__ src, size_t n,
                                                          float* __restrict__ sink) {
  size_t i = (size_t)blockIdx.x * kUtilBlock + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kUtilBlock;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 a = __builtin_nontemporal_load(src + i);
    u32x4 b = __builtin_nontemporal_load(src + i + stride);
    u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
    acc ^= c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n; i += stride) {
    u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  // a store that depends on every loaded word keeps the loads live; it
  // practically never fires
  if (acc == 0x9e3779b9u) sink[blockIdx.x % kReadSinkLen] = __uint_as_float(acc);
}

__global__ __launch_bounds__(kUtilBlock) void fill_kernel(u32x4* __restrict__ dst, size_t n,
                                                          uint32_t v) {
  size_t i = (size_t)blockIdx.x * kUtilBlock + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kUtilBlock;
  const u32x4 q = {v, v, v, v};
  for (; i < n; i += stride) dst[i] = q;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int stream_blocks() { return device_num_cus() * 8; }

}  // namespace

int device_num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_cus[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

// gfx950 parts (MI350 series) are built from 8 accelerator complex dies.
int device_num_xcds() { return 8; }

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3(stream_blocks()), dim3(kUtilBlock), 0, s,
                     reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_read(const void* src, size_t bytes, float* sink, hipStream_t s) {
  const size_t n = bytes / 16;
  const int blocks = std::min(stream_blocks(), kReadSinkLen);
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kUtilBlock), 0, s,
                     reinterpret_cast<const u32x4*>(src), n, sink);
  return hipGetLastError();
}

hipError_t launch_fill(void* dst, size_t bytes, uint32_t value, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(stream_blocks()), dim3(kUtilBlock), 0, s,
                     reinterpret_cast<u32x4*>(dst), n, value);
  return hipGetLastError();
}

}  // namespace moe
