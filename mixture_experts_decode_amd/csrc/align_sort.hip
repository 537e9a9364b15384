// MoE align-and-sort: group (token, slot) entries by expert, pad every
// expert's run to the grouped GEMM's block size.
//
// Structure after the align-and-sort article's D-C-P section (distributed
// concurrent counting, then the cumulative sums -- local unaligned, merged,
// aligned global, stored -- then parallel placement), re-planned for gfx950:
//  * count: every wavefront histograms its own contiguous range of entries in
//    a private LDS slice and stores the slice (no atomics to global memory,
//    no zero-initialised buffers, so the call is graph-capturable);
//  * prefix: one workgroup merges the per-wave histograms per expert into
//    exclusive per-wave bases, aligns each expert's total to the block size,
//    scans over experts, and writes offsets, block expert ids and the
//    sentinel padding;
//  * place: every wavefront walks its range again in order and gives each
//    entry its stable rank among equal ids (a match mask from per-bit
//    ballots, then a popcount), so the output is deterministic and ordered by
//    entry index inside every expert's run.
// Cross-workgroup data goes through L2 between launches (gfx950 has no
// on-chip workgroup-to-workgroup exchange; the article's CK/AITER section
// notes the same of CDNA3).  Up to 8192 entries one workgroup runs all three
// phases with the exchange in LDS (as_fused_kernel): one launch instead of
// three, the same results.

#include <algorithm>

#include "device.h"
#include "internal.h"
#include "mx_quant.h"

namespace moe {

namespace {

constexpr int kAsBlock = 256;
constexpr int kAsWaves = kAsBlock / kWave;
constexpr int kMaxWaves = 128;        // count/place wavefronts per call
constexpr int kPrefixBlock = 1024;
constexpr int kFusedWaves = kPrefixBlock / kWave;       // 16
constexpr int kFusedMaxEntries = kFusedWaves * 8 * kWave;   // 8192

struct AsArgs {
  const int32_t* ids;
  int T, k, slots, E, n_exp, bs, n;   // n = T*slots entries, n_exp = E + S
  int per_wave;                        // entries per wavefront (multiple of 64)
  int n_waves;
  int id_bits;                         // bits to tell experts apart
  int32_t* hist;                       // [n_waves][n_exp]
  int32_t* base;                       // [n_waves][n_exp]
  int32_t* sorted;
  int32_t* expert_ids;
  int32_t* offsets;
  int32_t* npp;
};

__device__ __forceinline__ int entry_expert(const AsArgs& a, int i) {
  int e;
  if (a.slots == a.k) {
    e = a.ids[i];
  } else {
    const int t = i / a.slots, j = i - t * a.slots;
    e = j < a.k ? a.ids[t * a.k + j] : a.E;
  }
  return (unsigned)e < (unsigned)a.n_exp ? e : 0;
}

__global__ __launch_bounds__(kAsBlock) void as_count_kernel(const AsArgs a) {
  __shared__ int s_hist[kAsWaves][kMaxExpertsTotal];
  const int lane = threadIdx.x & (kWave - 1);
  const int wl = threadIdx.x >> 6;
  const int w = blockIdx.x * kAsWaves + wl;
  if (w >= a.n_waves) return;
  int* h = s_hist[wl];
  for (int e = lane; e < a.n_exp; e += kWave) h[e] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int lo = w * a.per_wave;
  const int hi = min(lo + a.per_wave, a.n);
  for (int i = lo + lane; i < hi; i += kWave) atomicAdd(&h[entry_expert(a, i)], 1);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int32_t* out = a.hist + (size_t)w * a.n_exp;
  for (int e = lane; e < a.n_exp; e += kWave) out[e] = h[e];
}

// From the per-expert counts in s_cnt: pad every count to the block size,
// scan over experts into s_off (and s_off[n_exp] = total), then write the
// offsets, the padded total, the block -> expert map and the sentinel tails.
// Whole workgroup of kPrefixBlock threads; two barriers inside, s_off
// complete on return.
__device__ __forceinline__ void layout_phase(const AsArgs& a, const int* s_cnt, int* s_off,
                                             int* s_wtot) {
  const int tid = threadIdx.x;
  // padded counts, exclusive scan over experts (blocked: thread handles a run)
  const int per_t = (a.n_exp + kPrefixBlock - 1) / kPrefixBlock;
  const int e0 = tid * per_t, e1 = min(e0 + per_t, a.n_exp);
  int local = 0;
  for (int e = e0; e < e1; ++e) local += (s_cnt[e] + a.bs - 1) / a.bs * a.bs;
  // inclusive scan of `local` over the workgroup: each wavefront scans its
  // 64 values with lane shifts, wavefront 0 scans the wavefront totals
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  int incl = local;
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += v;
  }
  if (lane == kWave - 1) s_wtot[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    int t = lane < kPrefixBlock / kWave ? s_wtot[lane] : 0;
    for (int off = 1; off < kPrefixBlock / kWave; off <<= 1) {
      const int v = __shfl_up(t, off, kWave);
      if (lane >= off) t += v;
    }
    if (lane < kPrefixBlock / kWave) s_wtot[lane] = t;
  }
  __syncthreads();
  incl += wid ? s_wtot[wid - 1] : 0;
  int run = incl - local;
  for (int e = e0; e < e1; ++e) {
    s_off[e] = run;
    run += (s_cnt[e] + a.bs - 1) / a.bs * a.bs;
  }
  if (tid == kPrefixBlock - 1) s_off[a.n_exp] = incl;
  __syncthreads();
  const int total = s_off[a.n_exp];
  for (int e = tid; e <= a.n_exp; e += kPrefixBlock) a.offsets[e] = s_off[e];
  if (tid == 0) *a.npp = total;

  // block -> expert (binary search over the offsets)
  const int n_blocks = total / a.bs;
  for (int b = tid; b < n_blocks; b += kPrefixBlock) {
    const int pos = b * a.bs;
    int lo = 0, hi = a.n_exp - 1;          // last e with s_off[e] <= pos
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    a.expert_ids[b] = lo;
  }
  // sentinel tails: (expert, r) pairs with r < bs - 1
  const int padw = a.bs - 1;
  if (padw > 0) {
    for (int q = tid; q < a.n_exp * padw; q += kPrefixBlock) {
      const int e = q / padw, r = q - e * padw;
      const int c = s_cnt[e];
      const int p = (c + a.bs - 1) / a.bs * a.bs;
      if (c + r < p) a.sorted[s_off[e] + c + r] = a.n;
    }
  }
}

// One workgroup: per-expert merge over waves, alignment, expert scan.
__global__ __launch_bounds__(kPrefixBlock) void as_prefix_kernel(const AsArgs a) {
  __shared__ int s_part[kPrefixBlock];
  __shared__ int s_off[kMaxExpertsTotal + 1];
  __shared__ int s_cnt[kMaxExpertsTotal];
  __shared__ int s_wtot[kPrefixBlock / kWave];
  const int tid = threadIdx.x;
  // G threads per expert, each over a contiguous run of waves
  const int G = max(1, min(kPrefixBlock / a.n_exp, 8));
  const int per = (a.n_waves + G - 1) / G;

  for (int base_e = 0; base_e < a.n_exp; base_e += kPrefixBlock / G) {
    const int e = base_e + tid / G;
    const int g = tid % G;
    const bool act = tid / G < kPrefixBlock / G && e < a.n_exp;
    const int w0 = g * per, w1 = min(w0 + per, a.n_waves);
    int sum = 0;
    if (act)
      for (int w = w0; w < w1; ++w) sum += a.hist[(size_t)w * a.n_exp + e];
    s_part[tid] = sum;
    __syncthreads();
    if (act) {
      int pre = 0, tot = 0;
      for (int q = 0; q < G; ++q) {
        const int v = s_part[(tid / G) * G + q];
        if (q < g) pre += v;
        tot += v;
      }
      if (g == 0) s_cnt[e] = tot;
      // exclusive base of each wave within the expert (offset added later)
      int run = pre;
      for (int w = w0; w < w1; ++w) {
        const int c = a.hist[(size_t)w * a.n_exp + e];
        a.base[(size_t)w * a.n_exp + e] = run;
        run += c;
      }
    }
    __syncthreads();
  }

  layout_phase(a, s_cnt, s_off, s_wtot);
  // the per-wave bases stay relative to their expert's offset; the place
  // kernel adds the offset when it loads them
}

__device__ __forceinline__ void place_range(const AsArgs& a, int* ctr, int lo, int hi, int lane);

__global__ __launch_bounds__(kAsBlock) void as_place_kernel(const AsArgs a) {
  __shared__ int s_ctr[kAsWaves][kMaxExpertsTotal];
  const int lane = threadIdx.x & (kWave - 1);
  const int wl = threadIdx.x >> 6;
  const int w = blockIdx.x * kAsWaves + wl;
  if (w >= a.n_waves) return;
  int* ctr = s_ctr[wl];
  const int32_t* bse = a.base + (size_t)w * a.n_exp;
  for (int e = lane; e < a.n_exp; e += kWave) ctr[e] = bse[e] + a.offsets[e];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  place_range(a, ctr, w * a.per_wave, min(w * a.per_wave + a.per_wave, a.n), lane);
}

// Stable placement of entries [lo, hi) by one wavefront: ctr[e] (LDS) holds
// the next free slot of expert e in sorted order for this range.
__device__ __forceinline__ void place_range(const AsArgs& a, int* ctr, int lo, int hi, int lane) {
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int i0 = lo; i0 < hi; i0 += kWave) {
    const int i = i0 + lane;
    const bool valid = i < hi;
    const int e = valid ? entry_expert(a, i) : 0;
    unsigned long long peers = __ballot(valid);
    for (int b = 0; b < a.id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const unsigned long long m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    const int cnt = __popcll(peers);
    int dst = 0;
    if (valid) dst = ctr[e] + rank;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      a.sorted[dst] = i;
      if (rank == cnt - 1) ctr[e] = dst + 1;     // last of its group advances the counter
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
}

// Small batches: count, merge, layout and placement in one workgroup of
// kPrefixBlock threads (up to kFusedWaves wavefronts, each on its own
// contiguous range), all exchanged through LDS -- one launch, no global
// scratch.  Same results as the three-launch path.
__device__ __forceinline__ void as_fused_body(const AsArgs& a) {
  __shared__ int s_h[kFusedWaves][kMaxExpertsTotal];   // per-wave counts, then bases
  __shared__ int s_off[kMaxExpertsTotal + 1];
  __shared__ int s_cnt[kMaxExpertsTotal];
  __shared__ int s_wtot[kPrefixBlock / kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  for (int q = tid; q < kFusedWaves * a.n_exp; q += kPrefixBlock) s_h[q / a.n_exp][q % a.n_exp] = 0;
  __syncthreads();
  const int lo = w * a.per_wave, hi = min(lo + a.per_wave, a.n);
  if (w < a.n_waves)
    for (int i = lo + lane; i < hi; i += kWave) atomicAdd(&s_h[w][entry_expert(a, i)], 1);
  __syncthreads();
  // per expert: exclusive base of every wave's range inside the expert
  for (int e = tid; e < a.n_exp; e += kPrefixBlock) {
    int run = 0;
    for (int v = 0; v < a.n_waves; ++v) {
      const int c = s_h[v][e];
      s_h[v][e] = run;
      run += c;
    }
    s_cnt[e] = run;
  }
  __syncthreads();
  layout_phase(a, s_cnt, s_off, s_wtot);
  if (w < a.n_waves) {
    int* ctr = s_h[w];
    for (int e = lane; e < a.n_exp; e += kWave) ctr[e] += s_off[e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    place_range(a, ctr, lo, hi, lane);
  }
}

__global__ __launch_bounds__(kPrefixBlock) void as_fused_kernel(const AsArgs a) { as_fused_body(a); }

// The layer's grouped front end up to kFusedMaxEntries entries, in one
// launch: workgroup 0 sorts the entries (as above) while the others quantise
// the token rows to MXFP8, one wavefront per row.  The two steps do not
// depend on each other, so the quantisation runs in the sort's shadow; the
// outputs are those of the two separate calls.
template <bool XF32>
__global__ __launch_bounds__(kPrefixBlock) void front_end_kernel(const AsArgs a, const void* x,
                                                                 int H, uint8_t* xq, uint8_t* xs) {
  if (blockIdx.x == 0) {
    as_fused_body(a);
    return;
  }
  const int t = (blockIdx.x - 1) * kFusedWaves + (int)(threadIdx.x >> 6);
  if (t < a.T) quant_row<XF32>(x, t, H, xq, xs, threadIdx.x & (kWave - 1));
}

AsArgs make_args(const int32_t* ids, int T, int k, int E, int S, int bs) {
  AsArgs a{};
  a.ids = ids;
  a.T = T;
  a.k = k;
  a.slots = k + S;
  a.E = E;
  a.n_exp = E + S;
  a.bs = bs;
  a.n = T * a.slots;
  const int chunks = (a.n + kWave - 1) / kWave;
  const int per_chunks = std::max(1, (chunks + kMaxWaves - 1) / kMaxWaves);
  a.per_wave = per_chunks * kWave;
  a.n_waves = std::max(1, (a.n + a.per_wave - 1) / a.per_wave);
  int bits = 0;
  while ((1 << bits) < a.n_exp) ++bits;
  a.id_bits = bits;
  return a;
}

// one workgroup: at most kFusedWaves ranges of whole 64-entry chunks
void set_fused_ranges(AsArgs& a) {
  const int chunks = std::max(1, (a.n + kWave - 1) / kWave);
  a.per_wave = (chunks + kFusedWaves - 1) / kFusedWaves * kWave;
  a.n_waves = std::max(1, (a.n + a.per_wave - 1) / a.per_wave);
}

}  // namespace

size_t align_sort_workspace_bytes(int n_entries, int n_experts) {
  const int chunks = (n_entries + kWave - 1) / kWave;
  const int per_chunks = std::max(1, (chunks + kMaxWaves - 1) / kMaxWaves);
  const int per_wave = per_chunks * kWave;
  const int n_waves = std::max(1, (n_entries + per_wave - 1) / per_wave);
  return (size_t)2 * n_waves * n_experts * sizeof(int32_t);
}

hipError_t launch_align_sort(const int32_t* ids, int T, int k, int E, int S, int bs,
                             int32_t* sorted, int32_t* expert_ids, int32_t* offsets,
                             int32_t* npp, void* ws, hipStream_t s) {
  AsArgs a = make_args(ids, T, k, E, S, bs);
  a.sorted = sorted;
  a.expert_ids = expert_ids;
  a.offsets = offsets;
  a.npp = npp;
  if (a.n <= kFusedMaxEntries) {
    set_fused_ranges(a);
    hipLaunchKernelGGL(as_fused_kernel, dim3(1), dim3(kPrefixBlock), 0, s, a);
    return hipGetLastError();
  }
  a.hist = reinterpret_cast<int32_t*>(ws);
  a.base = a.hist + (size_t)a.n_waves * a.n_exp;
  const int blocks = (a.n_waves + kAsWaves - 1) / kAsWaves;
  hipLaunchKernelGGL(as_count_kernel, dim3(blocks), dim3(kAsBlock), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(as_prefix_kernel, dim3(1), dim3(kPrefixBlock), 0, s, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(as_place_kernel, dim3(blocks), dim3(kAsBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_front_end(const int32_t* ids, int T, int k, int E, int S, int bs,
                            int32_t* sorted, int32_t* expert_ids, int32_t* offsets, int32_t* npp,
                            void* ws, const void* x, int x_dtype, int H, uint8_t* xq, uint8_t* xs,
                            hipStream_t s) {
  AsArgs a = make_args(ids, T, k, E, S, bs);
  if (a.n > kFusedMaxEntries || T == 0 || x_dtype == MOE_DT_F32) {
    hipError_t err = launch_align_sort(ids, T, k, E, S, bs, sorted, expert_ids, offsets, npp, ws, s);
    if (err != hipSuccess) return err;
    return launch_quant_rows(x, x_dtype, T, H, xq, xs, s);
  }
  a.sorted = sorted;
  a.expert_ids = expert_ids;
  a.offsets = offsets;
  a.npp = npp;
  set_fused_ranges(a);
  const dim3 grid(1 + (T + kFusedWaves - 1) / kFusedWaves), block(kPrefixBlock);
  hipLaunchKernelGGL(front_end_kernel<false>, grid, block, 0, s, a, x, H, xq, xs);
  return hipGetLastError();
}

}  // namespace moe
