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

// One 16-byte element per thread over a grid that covers the buffer: every
// wavefront issues one load (and one store) and retires, which keeps the most
// requests in flight (measured on MI355X: 6.1 TB/s read + write for 2 GiB,
// against 4.7 TB/s for a grid-stride loop and 5.0 TB/s for a device memcpy).
__global__ __launch_bounds__(kUtilBlock) void copy_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, size_t n) {
  const size_t i = (size_t)blockIdx.x * kUtilBlock + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

__global__ __launch_bounds__(kUtilBlock) void read_kernel(const u32x4* __restrict__ src, size_t n,
                                                          float* __restrict__ sink) {
  const size_t i = (size_t)blockIdx.x * kUtilBlock + threadIdx.x;
  if (i >= n) return;
  const u32x4 a = src[i];
  const uint32_t acc = a[0] ^ a[1] ^ a[2] ^ a[3];
  // a store that depends on every loaded word keeps the load live; it
  // practically never fires
  if (acc == 0x9e3779b9u) sink[blockIdx.x % kReadSinkLen] = __uint_as_float(acc);
}

__global__ __launch_bounds__(kUtilBlock) void fill_kernel(u32x4* __restrict__ dst, size_t n,
                                                          uint32_t v) {
  const size_t i = (size_t)blockIdx.x * kUtilBlock + threadIdx.x;
  if (i < n) dst[i] = u32x4{v, v, v, v};
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

// blocks covering n 16-byte elements, one per thread
unsigned cover_blocks(size_t n) { return (unsigned)((n + kUtilBlock - 1) / kUtilBlock); }

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
  if ((n + kUtilBlock - 1) / kUtilBlock > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3(cover_blocks(n)), dim3(kUtilBlock), 0, s,
                     reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_read(const void* src, size_t bytes, float* sink, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  if ((n + kUtilBlock - 1) / kUtilBlock > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3(cover_blocks(n)), dim3(kUtilBlock), 0, s,
                     reinterpret_cast<const u32x4*>(src), n, sink);
  return hipGetLastError();
}

hipError_t launch_fill(void* dst, size_t bytes, uint32_t value, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  if ((n + kUtilBlock - 1) / kUtilBlock > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fill_kernel, dim3(cover_blocks(n)), dim3(kUtilBlock), 0, s,
                     reinterpret_cast<u32x4*>(dst), n, value);
  return hipGetLastError();
}

}  // namespace moe
