// Router front-end: gating scores -> top-k expert ids and routing weights.
//
// The align-and-sort article's background section activates the experts with
// the top-k gating scores, a per-expert bias added for the selection in
// DeepSeek V3/R1; its FasterTransformer section names the fused top-k gating
// softmax.  Here: key = score + bias in FP32, the k largest keys (equal keys
// to the lower expert index) in descending order, weights = softmax over the
// selected raw scores.
//
// One wavefront per token.  Lane l holds experts l, l + 64, ... as 64-bit
// candidates ordered like (key, -index): the key's bits mapped to an unsigned
// order in the high word, the complement of the index in the low word.  Each
// of the k rounds takes a wave maximum (DPP and row swaps) and retires the winner
// in its owner lane.  Lane j then keeps winner j and its score for the
// softmax, which subtracts the selected maximum and sums with a wave
// reduction.

#include "device.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kRouteBlock = 256;

// Wave maximum of 64-bit (key, index) candidates: the largest key word,
// then the largest index word among the lanes holding it.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
  const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
  return ((uint64_t)hi << 32) | lo;
}

// Wave maximum of a float (finite or -inf inputs), every lane gets it.
__device__ __forceinline__ float wave_max_f32(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  const uint32_t m = wave_max_u32(o);
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7fffffffu) : ~m);
}

// Monotone map of a finite float to uint32 (-0 and +0 map alike).
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int PER>
__global__ __launch_bounds__(kRouteBlock) void topk_route_kernel(
    const float* __restrict__ scores, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (kRouteBlock / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = scores + (size_t)t * E;
  uint64_t cand[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    if (e < E) {
      const float key = bias ? row[e] + bias[e] : row[e];
      cand[i] = ((uint64_t)ordered_bits(key) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
    } else {
      cand[i] = 0;   // below every real candidate
    }
  }
  int mine = -1;   // winner of round `lane`
  for (int j = 0; j < k; ++j) {
    uint64_t best = cand[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) best = cand[i] > best ? cand[i] : best;
    best = wave_max_u64(best);
    const int win = (int)(0xffffffffu - (uint32_t)best);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane + kWave * i == win) cand[i] = 0;
    if (lane == j) mine = win;
  }
  const float s = mine >= 0 ? row[mine] : -INFINITY;
  const float m = wave_max_f32(s);
  const float p = mine >= 0 ? expf(s - m) : 0.0f;
  const float sum = wave_sum(p);
  if (mine >= 0) {
    ids[(size_t)t * k + lane] = mine;
    wts[(size_t)t * k + lane] = p / sum;
  }
}

}  // namespace

hipError_t launch_topk_route(const float* scores, const float* bias, int T, int E, int k,
                             int32_t* ids, float* wts, hipStream_t s) {
  const dim3 grid((T + kRouteBlock / kWave - 1) / (kRouteBlock / kWave)), block(kRouteBlock);
#define MOE_RT(P) \
  hipLaunchKernelGGL((topk_route_kernel<P>), grid, block, 0, s, scores, bias, T, E, k, ids, wts)
  if (E <= 64) MOE_RT(1);
  else if (E <= 128) MOE_RT(2);
  else if (E <= 256) MOE_RT(4);
  else if (E <= 512) MOE_RT(8);
  else MOE_RT(16);
#undef MOE_RT
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Routing check: how many routed ids lie outside [0, E), and the first one.
// One workgroup walks all T*k ids and writes the two numbers once, so nothing
// has to be cleared before it (no memset, safe inside a captured graph) and
// the result does not depend on any scheduling.
// ---------------------------------------------------------------------------

namespace {

constexpr int kCheckBlock = 1024;

__global__ __launch_bounds__(kCheckBlock) void check_routing_kernel(const int32_t* __restrict__ ids,
                                                                    int n, int E,
                                                                    int32_t* __restrict__ out) {
  __shared__ int s_cnt[kCheckBlock / kWave];
  __shared__ int s_first[kCheckBlock / kWave];
  int cnt = 0, first = n;
  for (long long i = threadIdx.x; i < n; i += kCheckBlock) {
    if ((unsigned)ids[i] >= (unsigned)E) {
      ++cnt;
      first = min(first, (int)i);
    }
  }
  for (int off = kWave / 2; off > 0; off >>= 1) {
    cnt += __shfl_xor(cnt, off, kWave);
    first = min(first, __shfl_xor(first, off, kWave));
  }
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    s_cnt[w] = cnt;
    s_first[w] = first;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0, f = n;
    for (int q = 0; q < kCheckBlock / kWave; ++q) {
      c += s_cnt[q];
      f = min(f, s_first[q]);
    }
    out[0] = c;
    out[1] = f < n ? f : -1;
  }
}

}  // namespace

hipError_t launch_check_routing(const int32_t* ids, int n, int E, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(check_routing_kernel, dim3(1), dim3(kCheckBlock), 0, s, ids, n, E, out);
  return hipGetLastError();
}

}  // namespace moe
