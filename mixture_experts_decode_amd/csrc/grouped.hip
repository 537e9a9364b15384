// Expert-centric (grouped) path: MXFP8 quantisation of each token row once,
// grouped gate_up / down GEMMs on gfx950 block-scaled MFMA (the gate_up
// GEMM's activation loads follow the align-sort order to the token rows),
// ordered combine.

#include "device.h"
#include "internal.h"
#include "mx_quant.h"

namespace moe {

namespace {

constexpr int kGqBlock = 256;

// One wavefront per token row; each lane quantises whole 32-element blocks.
// Every token is quantised once, whatever number of slots routes it: the
// gate_up GEMM reads a sorted row's activations from its token's row.
template <bool XF32>
__global__ __launch_bounds__(kGqBlock) void quant_rows_kernel(const void* __restrict__ x, int T,
                                                              int H, uint8_t* __restrict__ xq,
                                                              uint8_t* __restrict__ xs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (kGqBlock / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;
  quant_row<XF32>(x, t, H, xq, xs, lane);
}

// Slots are FP32 (decode path) or BF16 (grouped path); the sum is FP32 in
// slot order either way.
template <bool YBF16, bool SBF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ so, int T,
                                                      int slots, int H, void* __restrict__ y) {
  const int h4 = H >> 2;
  const size_t n = (size_t)T * h4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t t = i / h4;
    const size_t c = i - t * h4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // up to eight slots' loads are issued before their adds (in slot order)
    for (int j0 = 0; j0 < slots; j0 += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        if (j < slots) {
          if constexpr (SBF16) {
            const uint2 q = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(so) +
                                                           (t * slots + j) * H)[c];
            v[u] = make_float4(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y));
          } else {
            v[u] = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(so) +
                                                   (t * slots + j) * H)[c];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u < slots) {
          acc.x += v[u].x;
          acc.y += v[u].y;
          acc.z += v[u].z;
          acc.w += v[u].w;
        }
      }
    }
    if constexpr (YBF16) {
      uint2 o;
      o.x = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
      o.y = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
      reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + t * H)[c] = o;
    } else {
      reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + t * H)[c] = acc;
    }
  }
}

}  // namespace

hipError_t launch_quant_rows(const void* x, int x_dtype, int T, int H, uint8_t* xq, uint8_t* xs,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int rows_per_block = kGqBlock / kWave;
  const int blocks = (T + rows_per_block - 1) / rows_per_block;
  if (x_dtype == MOE_DT_F32)
    hipLaunchKernelGGL(quant_rows_kernel<true>, dim3(blocks), dim3(kGqBlock), 0, s, x, T, H, xq, xs);
  else
    hipLaunchKernelGGL(quant_rows_kernel<false>, dim3(blocks), dim3(kGqBlock), 0, s, x, T, H, xq,
                       xs);
  return hipGetLastError();
}

hipError_t launch_combine(const void* slot_out, int slot_dtype, int T, int slots, int H, void* y,
                          int y_dtype, hipStream_t s) {
  if (H % 4) return hipErrorNotSupported;
  const size_t n = (size_t)T * (H / 4);
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, (size_t)device_num_cus() * 16);
  const bool yb = y_dtype == MOE_DT_BF16, sb = slot_dtype == MOE_DT_BF16;
  if (yb && sb)
    hipLaunchKernelGGL((combine_kernel<true, true>), dim3(blocks), dim3(256), 0, s, slot_out, T, slots, H, y);
  else if (yb)
    hipLaunchKernelGGL((combine_kernel<true, false>), dim3(blocks), dim3(256), 0, s, slot_out, T, slots, H, y);
  else if (sb)
    hipLaunchKernelGGL((combine_kernel<false, true>), dim3(blocks), dim3(256), 0, s, slot_out, T, slots, H, y);
  else
    hipLaunchKernelGGL((combine_kernel<false, false>), dim3(blocks), dim3(256), 0, s, slot_out, T, slots, H, y);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// grouped GEMMs on v_mfma_scale_f32_32x32x64_f8f6f4
//
// A workgroup of 4 or 8 wavefronts computes a BM x BN tile: BM sorted rows (one
// align-sort block, hence one expert) against BN weight rows.  In gate_up the
// sorted rows' activations are the quantised rows of their tokens, fetched
// through sorted_token_ids by the same direct-to-LDS loads (no gathered copy
// exists); in down they are the sorted rows of h that gate_up wrote.  Both operand
// tiles travel HBM -> LDS by direct-to-LDS loads (global_load_lds_dwordx4),
// in NS stages of 64 * KSTEPS K, so NS-1 stages are in flight while one is
// consumed and no registers are spent on staging.  An LDS row holds one
// stage of a matrix row with its 16-byte chunks XOR-swizzled by the row
// index: every DMA instruction still writes 1 KB contiguously (whole rows),
// and the MFMA operand reads of 8 or 16 consecutive rows land on distinct
// banks.  The MX scales ride along (one dword = four 32-K blocks per row).
// Weights are the MFMA row operand and activations the column operand, so a
// lane ends up with 16 outputs of one sorted row.  The grid is persistent:
// the tiles (M-block, N-tile) are counted on the device from the padded
// total, split evenly over the XCDs and walked in groups of M-blocks, so that
// concurrent workgroups on one XCD share activation and weight rows in L2.
// The L2 -> CU path (about 12.5 TB/s over the chip in whole 128-byte lines,
// measured) rather than the matrix cores bounds the large-batch tiles.
// ---------------------------------------------------------------------------

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLdsBytes = 160 * 1024;    // gfx950 LDS per workgroup
constexpr int kGroupM = 4;               // M-blocks per raster group

struct GemmArgs {
  const uint8_t* a;        // gate_up: token rows [T][K] E4M3; down: sorted rows of h's hi term [cap][K]
  const uint8_t* as;       // [T or cap][K/32] E8M0
  const uint8_t* a_lo;     // down: lo term of h [cap][K]
  const uint8_t* as_lo;    // down: [cap][K/32]
  const uint8_t* b;        // expert weights, rows of K (E4M3 or packed E2M1)
  const void* bs;          // weight scales (E8M0 bytes or float 128x128 tiles)
  const int32_t* expert_ids;
  const int32_t* npp;
  const int32_t* sorted;   // entry of each sorted row (gate_up: its token row; down: its slot)
  const float* wts;        // down: routing weights
  uint8_t* hq;             // gate_up out [2][cap][I]: hi term, then lo term
  uint8_t* hs;             // gate_up out [2][cap][I/32]
  int cap;
  uint16_t* out;           // down out: slot_out [T*slots][H] BF16
  int K, N;                // reduction length, output columns (neurons or H)
  int I, H;
  int b_row_bytes;
  int rows_per_expert;     // 2I (gate_up) or H (down)
  int n_ntiles;            // tiles along N
  int k, slots, sentinel;
  int nxcd;
};

__device__ __forceinline__ void dma16(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

__device__ __forceinline__ void dma4(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// Wait until at most N vector-memory operations of this wavefront are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Workgroup barrier without the memory-model fence of __syncthreads (which
// would drain every DMA in flight).  This wavefront's LDS reads complete
// before it arrives, so no buffer is overwritten under a pending read.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS slot of 16-byte chunk c of row r is c ^ swz<P>(r) for rows of P chunks
// (P = 8, 4, 2: rows of 128, 64, 32 bytes): a bijection per row that spreads
// 8 (and 16) consecutive rows reading the same chunk over distinct banks.
template <int P>
__device__ __forceinline__ int swz(int r) {
  if constexpr (P == 8) return (r & 7) ^ ((r >> 3) & 1);
  else if constexpr (P == 4) return ((r >> 1) ^ (r >> 3)) & 3;
  else if constexpr (P == 16) return r & 15;
  else return ((r >> 2) ^ (r >> 3)) & 1;
}

// Max of x over lanes l and l ^ 32.
__device__ __forceinline__ float pair32_max(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int BFMT, bool GATEUP, int BM, int BN, int WM, int WN, int KSTEPS>
struct GemmShape {
  static constexpr int TERMS = GATEUP ? 1 : 2;    // down reads h as hi + lo
  static constexpr bool FP4 = BFMT == W_MXFP4;
  static constexpr bool T128 = BFMT == W_FP8B128;
  static constexpr int KSTAGE = 64 * KSTEPS;       // K elements per stage
  static constexpr int ARB = KSTAGE;               // activation bytes per row and stage
  static constexpr int BRB = FP4 ? KSTAGE / 2 : KSTAGE;
  static constexpr int AP = ARB / 16, BP = BRB / 16;   // 16-byte chunks per LDS row
  static constexpr int WROWS = BM / WM;            // wavefront sub-tile
  static constexpr int WCOLS = BN / WN;
  static constexpr int MF = WROWS / 32;
  static constexpr int NF = WCOLS / 32;
  static constexpr int A_BYTES = TERMS * BM * ARB;
  static constexpr int B_BYTES = BN * BRB;
  // activation scales: shared by the workgroup when every wavefront covers
  // all BM = 128 rows (wavefront w loads rows 32w..32w+31 into a 64-dword
  // slot, upper half duplicated), else one slice per wavefront of its rows
  static constexpr int WAVES = WM * WN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr bool AS_COOP = WM == 1 && BM == 128 && WAVES == 4;
  static constexpr int SA = WROWS < 64 ? 64 : WROWS;
  // scale dwords (four 32-K blocks each) per row and stage; a 64-K stage
  // reads half a dword
  static constexpr int SD = KSTEPS >= 2 ? KSTEPS / 2 : 1;
  static constexpr int AS1 = AS_COOP ? TERMS * 4 * 64 * 4 : WAVES * TERMS * SA * 4;
  static constexpr int AS_BYTES = SD * AS1;
  static constexpr int SB = T128 ? 64 : (WCOLS < 64 ? 64 : WCOLS);   // per wavefront
  static constexpr int BS1 = WAVES * SB * 4;
  static constexpr int BS_BYTES = SD * BS1;
  static constexpr int STAGE = A_BYTES + B_BYTES + AS_BYTES + BS_BYTES;
  static constexpr int NS_FIT = kLdsBytes / STAGE;
  static constexpr int NS = NS_FIT > 4 ? 4 : NS_FIT;
  static constexpr int A_INSTR = A_BYTES / 1024 / WAVES;   // per wavefront
  static constexpr int B_INSTR = B_BYTES / 1024 / WAVES;
  static constexpr int SA_INSTR = AS_COOP ? TERMS : TERMS * (SA / 64);
  static constexpr int SB_INSTR = SB / 64;
  static constexpr int L = A_INSTR + B_INSTR + SD * (SA_INSTR + SB_INSTR);   // DMA ops per stage
  static_assert(KSTEPS == 1 || KSTEPS == 2 || (KSTEPS == 4 && FP4), "stage depth");
  static_assert(WAVES == 4 || WAVES == 8, "four or eight wavefronts");
  static_assert(WROWS % 32 == 0 && WCOLS % 32 == 0, "whole fragments");
  static_assert(!GATEUP || NF % 2 == 0, "gate and up fragments pair up");
  static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0, "whole DMA rounds");
  static_assert(NS >= 2, "double buffering fits");
  static_assert((NS - 2) * L < 64, "vmcnt range");
};

template <int BFMT, bool GATEUP, int BM, int BN, int WM, int WN, int KSTEPS>
__global__ __launch_bounds__(64 * WM * WN) void grouped_gemm_kernel(const GemmArgs g) {
  using S = GemmShape<BFMT, GATEUP, BM, BN, WM, WN, KSTEPS>;
  constexpr int MF = S::MF, NF = S::NF, TERMS = S::TERMS, NS = S::NS;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * S::STAGE];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
  const int r32 = lane & 31, h = lane >> 5;
  const int wm = w / WN, wn = w % WN;

  const int nx = g.nxcd;
  const int xcd = blockIdx.x % nx, local = blockIdx.x / nx, per_x = gridDim.x / nx;
  const int n_mb = *g.npp / BM;
  const int total = n_mb * g.n_ntiles;
  const int chunk = (total + nx - 1) / nx;
  const int t_end = min(total, (xcd + 1) * chunk);
  const int nst = g.K / S::KSTAGE;
  const int k_blocks = g.K >> 5;
  const int k_tiles = g.K >> 7;

  // tile row of the weight operand -> weight row inside the expert
  auto b_row = [&](int nt, int trow) -> int {
    if constexpr (GATEUP) {
      const int proj = trow >= BN / 2 ? 1 : 0;
      const int n = min(nt * (BN / 2) + trow - proj * (BN / 2), g.N - 1);
      return proj * g.I + n;
    } else {
      return min(nt * BN + trow, g.N - 1);
    }
  };
  // tile row of weight row i (0 <= i < WCOLS) of this wavefront; fragment f
  // covers i in [32f, 32f + 32)
  auto wave_brow = [&](int i) -> int {
    if constexpr (GATEUP) {
      const int f = i >> 5, r = i & 31;
      return f < NF / 2 ? wn * (S::WCOLS / 2) + 32 * f + r
                        : BN / 2 + wn * (S::WCOLS / 2) + 32 * (f - NF / 2) + r;
    } else {
      return wn * S::WCOLS + i;
    }
  };

  // lane-constant LDS read offsets of the MFMA operands, per K step and half:
  // an 8-bit operand lane holds bytes [16h, 16h+16) and [32+16h, 32+16h+16)
  // of the 64-K step, an E2M1 lane bytes [16h, 16h+16) of its 32-byte step
  int a_off[KSTEPS][2], b_off[KSTEPS][2];
#pragma unroll
  for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      a_off[st][q] = r32 * S::ARB + (((4 * st + 2 * q + h) ^ swz<S::AP>(r32)) << 4);
      b_off[st][q] = S::FP4 ? r32 * S::BRB + (((2 * st + h) ^ swz<S::BP>(r32)) << 4)
                            : r32 * S::BRB + (((4 * st + 2 * q + h) ^ swz<S::BP>(r32)) << 4);
    }

  // token row of sorted row r (gate_up): the entry's token, or token 0 for
  // a padding row
  auto token_of = [&](int r) -> int {
    const int ent = g.sorted[r];
    return (unsigned)ent < (unsigned)g.sentinel ? ent / g.slots : 0;
  };

  // per-tile state, set by setup(t) for the tile whose loads are queued
  constexpr int AR_I = 1024 / S::ARB, BR_I = 1024 / S::BRB;   // rows per DMA instruction
  int row0 = 0, nt = 0;
  const uint8_t* a_base0 = g.a;
  const uint8_t* a_base1 = g.a;
  const uint8_t* b_base = g.b;
  const uint8_t* sa_base0 = g.as;
  const uint8_t* sa_base1 = g.as;
  const uint8_t* sb_base = reinterpret_cast<const uint8_t*>(g.bs);
  uint32_t a_src[S::A_INSTR];
  uint32_t b_src[S::B_INSTR];
  uint32_t sa_src[S::SA_INSTR];
  int sa_dst[S::SA_INSTR];
  uint32_t sb_src[S::SB_INSTR];

  auto setup = [&](int t) {
    const int gsz = kGroupM * g.n_ntiles;
    const int grp = t / gsz;
    const int rem = t - grp * gsz;
    const int gm = min(kGroupM, n_mb - grp * kGroupM);
    nt = rem / gm;
    // uniform by construction; said so, the expert id is a scalar load
    const int mb = __builtin_amdgcn_readfirstlane(grp * kGroupM + (rem - nt * gm));
    const int e = g.expert_ids[mb];
    row0 = mb * BM;
    // the per-lane DMA offsets are recomputed for every tile (a few VALU
    // operations) rather than hoisted out of the tile loop and spilled
    int ln = lane;
    asm volatile("" : "+v"(ln));

    // ---- DMA sources: a uniform base per operand (advanced by the stage)
    // plus a 32-bit per-lane offset that stays fixed for the whole tile
    // gate_up reads each sorted row's activations from its token's row
    // (padding rows read token 0; their outputs are never used); down reads
    // the sorted rows of h that gate_up wrote
    a_base0 = GATEUP ? g.a : g.a + (size_t)row0 * g.K;
    a_base1 = TERMS > 1 ? g.a_lo + (size_t)row0 * g.K : a_base0;
    b_base = g.b + (size_t)e * g.rows_per_expert * g.b_row_bytes;
#pragma unroll
    for (int i = 0; i < S::A_INSTR; ++i) {
      const int j = (w + S::WAVES * i) % (BM / AR_I);
      const int row = AR_I * j + ln / S::AP;
      const uint32_t src_row = GATEUP ? (uint32_t)token_of(row0 + row) : (uint32_t)row;
      a_src[i] = src_row * (uint32_t)g.K + (uint32_t)(((ln % S::AP) ^ swz<S::AP>(row)) << 4);
    }
#pragma unroll
    for (int i = 0; i < S::B_INSTR; ++i) {
      const int row = BR_I * (w + S::WAVES * i) + ln / S::BP;
      b_src[i] = (uint32_t)(b_row(nt, row) * g.b_row_bytes + (((ln % S::BP) ^ swz<S::BP>(row)) << 4));
    }
    sa_base0 = GATEUP ? g.as : g.as + (size_t)row0 * k_blocks;
    sa_base1 = TERMS > 1 ? g.as_lo + (size_t)row0 * k_blocks : sa_base0;
    sb_base =
        S::T128 ? reinterpret_cast<const uint8_t*>(g.bs) + (size_t)e * (g.rows_per_expert >> 7) * k_tiles * 4
                : reinterpret_cast<const uint8_t*>(g.bs) + (size_t)e * g.rows_per_expert * k_blocks;
#pragma unroll
    for (int q = 0; q < S::SA_INSTR; ++q) {
      int srow;
      if constexpr (S::AS_COOP) {
        srow = 32 * w + (ln & 31);
        sa_dst[q] = (q * 256 + w * 64) * 4;                // term q, slot w
      } else {
        const int tm = q / (S::SA / 64), u = q % (S::SA / 64);
        const int rw = S::WROWS >= 64 ? 64 * u + ln : ln % S::WROWS;
        srow = wm * S::WROWS + rw;
        sa_dst[q] = ((w * TERMS + tm) * S::SA + 64 * u) * 4;
      }
      const uint32_t src_row = GATEUP ? (uint32_t)token_of(row0 + srow) : (uint32_t)srow;
      sa_src[q] = src_row * (uint32_t)k_blocks;
    }
#pragma unroll
    for (int u = 0; u < S::SB_INSTR; ++u) {
      if constexpr (S::T128) {
        sb_src[u] = (uint32_t)((b_row(nt, wave_brow(32 * (ln % NF))) >> 7) * k_tiles * 4);
      } else {
        const int i = S::WCOLS >= 64 ? 64 * u + ln : ln % S::WCOLS;
        sb_src[u] = (uint32_t)(b_row(nt, wave_brow(i)) * k_blocks);
      }
    }
  };

  // stage s reads the SD scale dwords from the one holding K block 2 * s * KSTEPS
  auto issue = [&](int s, int buf) {
    uint8_t* base = lds + buf * S::STAGE;
    const int ks = s * S::KSTAGE;                   // first K element of the stage
#pragma unroll
    for (int i = 0; i < S::A_INSTR; ++i) {
      const int j = w + S::WAVES * i;               // WG instruction: plane j / (BM / AR_I)
      const uint8_t* src = (j >= BM / AR_I ? a_base1 : a_base0) + ks;
      dma16(src + a_src[i], base + (j / (BM / AR_I)) * BM * S::ARB + (j % (BM / AR_I)) * 1024);
    }
#pragma unroll
    for (int i = 0; i < S::B_INSTR; ++i)
      dma16(b_base + (S::FP4 ? ks / 2 : ks) + b_src[i], base + S::A_BYTES + (w + S::WAVES * i) * 1024);
    const int sdw = (ks >> 7) * 4;                  // byte offset of the scale dword
    uint8_t* as_lds = base + S::A_BYTES + S::B_BYTES;
#pragma unroll
    for (int d = 0; d < S::SD; ++d)
#pragma unroll
      for (int q = 0; q < S::SA_INSTR; ++q) {
        const int tm = S::AS_COOP ? q : q / (S::SA / 64);
        dma4((tm ? sa_base1 : sa_base0) + sdw + 4 * d + sa_src[q], as_lds + d * S::AS1 + sa_dst[q]);
      }
    uint8_t* bs_lds = as_lds + S::AS_BYTES + w * S::SB * 4;
#pragma unroll
    for (int d = 0; d < S::SD; ++d)
#pragma unroll
      for (int u = 0; u < S::SB_INSTR; ++u)
        dma4(sb_base + (S::T128 ? (ks >> 7) * 4 : sdw + 4 * d) + sb_src[u],
             bs_lds + d * S::BS1 + 64 * u * 4);
  };

  // acc[m][f]: 32 weight rows of fragment f (MFMA rows) x 32 sorted rows of
  // fragment m (MFMA columns)
  f32x16 acc[MF][NF];
#pragma unroll
  for (int m = 0; m < MF; ++m)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[m][f] = f32x16{0};
  f32x16 part[S::T128 ? MF : 1][S::T128 ? NF : 1];
  if constexpr (S::T128) {
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
      for (int f = 0; f < NF; ++f) part[m][f] = f32x16{0};
  }

  auto compute = [&](int s, int buf) {
    const uint8_t* base = lds + buf * S::STAGE;
    const uint8_t* at = base + wm * S::WROWS * S::ARB;
    const uint8_t* bt = base + S::A_BYTES;
    const uint32_t* as_lds = reinterpret_cast<const uint32_t*>(base + S::A_BYTES + S::B_BYTES);
    const uint32_t* bs_lds = as_lds + S::AS_BYTES / 4 + w * S::SB;
    uint32_t sa[S::SD][TERMS][MF];
#pragma unroll
    for (int d = 0; d < S::SD; ++d)
#pragma unroll
      for (int tm = 0; tm < TERMS; ++tm)
#pragma unroll
        for (int m = 0; m < MF; ++m) {
          if constexpr (S::AS_COOP) sa[d][tm][m] = as_lds[d * S::AS1 / 4 + tm * 256 + m * 64 + r32];
          else sa[d][tm][m] = as_lds[d * S::AS1 / 4 + (w * TERMS + tm) * S::SA + 32 * m + r32];
        }
    uint32_t sb[S::SD][NF];
    float tsc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if constexpr (S::T128) {
        tsc[f] = __uint_as_float(bs_lds[f]);
        sb[0][f] = 0x7f7f7f7fu;
      } else {
#pragma unroll
        for (int d = 0; d < S::SD; ++d) sb[d][f] = bs_lds[d * S::BS1 / 4 + 32 * f + r32];
      }
    }
    // byte of the scale dword for K step st of this stage, K block h
    const int sbyte0 = KSTEPS == 2 ? 0 : 2 * (s & 1);
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      const int ds = KSTEPS >= 2 ? st >> 1 : 0;        // scale dword of this K step
      const int sh = KSTEPS >= 2 ? 8 * (2 * (st & 1) + h) : 8 * (sbyte0 + h);
      i32x8 bf[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const uint8_t* br = bt + wave_brow(32 * f) * S::BRB;
        if constexpr (S::FP4) {
          const u32x4 q0 = *reinterpret_cast<const u32x4*>(br + b_off[st][0]);
          bf[f] = i32x8{(int)q0[0], (int)q0[1], (int)q0[2], (int)q0[3], 0, 0, 0, 0};
        } else {
          const u32x4 q0 = *reinterpret_cast<const u32x4*>(br + b_off[st][0]);
          const u32x4 q1 = *reinterpret_cast<const u32x4*>(br + b_off[st][1]);
          bf[f] = i32x8{(int)q0[0], (int)q0[1], (int)q0[2], (int)q0[3],
                        (int)q1[0], (int)q1[1], (int)q1[2], (int)q1[3]};
        }
      }
#pragma unroll
      for (int tm = 0; tm < TERMS; ++tm) {
#pragma unroll
        for (int m = 0; m < MF; ++m) {
          const uint8_t* ar = at + tm * BM * S::ARB + m * 32 * S::ARB;
          const u32x4 q0 = *reinterpret_cast<const u32x4*>(ar + a_off[st][0]);
          const u32x4 q1 = *reinterpret_cast<const u32x4*>(ar + a_off[st][1]);
          const i32x8 af = {(int)q0[0], (int)q0[1], (int)q0[2], (int)q0[3],
                            (int)q1[0], (int)q1[1], (int)q1[2], (int)q1[3]};
          const int sca = (int)((sa[ds][tm][m] >> sh) & 0xffu);
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const int scb = (int)((sb[ds][f] >> sh) & 0xffu);
            // weights as the first (row) operand, activations as the second
            if constexpr (S::T128) {
              part[m][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  bf[f], af, part[m][f], 0, 0, 0, scb, 0, sca);
            } else {
              acc[m][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  bf[f], af, acc[m][f], S::FP4 ? 4 : 0, 0, 0, scb, 0, sca);
            }
          }
        }
      }
    }
    if constexpr (S::T128) {
      // a 128-wide K tile is complete: promote it with its float scale
      if (KSTEPS == 2 || (s & 1)) {
#pragma unroll
        for (int m = 0; m < MF; ++m)
#pragma unroll
          for (int f = 0; f < NF; ++f) {
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[m][f][q] = fmaf(part[m][f][q], tsc[f], acc[m][f][q]);
            part[m][f] = f32x16{0};
          }
      }
    }
  };

  int t = xcd * chunk + local;
  if (t < t_end) {
    setup(t);
    for (int s = 0; s < min(NS - 1, nst); ++s) issue(s, s);
  }
  while (t < t_end) {
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[m][f] = f32x16{0};

    // ---- pipeline: NS-1 stages in flight (the first ones were queued
    // before the previous tile's epilogue)
    int buf = 0;
    for (int s = 0; s < nst; ++s) {
      if (s + NS - 1 <= nst) wait_vmem<(NS - 2) * S::L>();
      else wait_vmem<0>();
      wg_barrier();
      if (s + NS - 1 < nst) {
        const int nb = buf == 0 ? NS - 1 : buf - 1;     // (s + NS - 1) % NS
        issue(s + NS - 1, nb);
      }
      compute(s, buf);
      buf = buf + 1 == NS ? 0 : buf + 1;
    }

    // ---- next tile: its first stages are queued before this tile's
    // epilogue, which then overlaps them.  Epilogue values that come from
    // memory are read first: vector memory completes in issue order, so a
    // later wait for them would also wait for the queued stages.
    const int tile_row0 = row0, tile_nt = nt;
    int ent[GATEUP ? 1 : MF];
    float wgt[GATEUP ? 1 : MF];
    if constexpr (!GATEUP) {
#pragma unroll
      for (int m = 0; m < MF; ++m) ent[m] = g.sorted[row0 + wm * S::WROWS + m * 32 + r32];
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        const bool real = ent[m] >= 0 && ent[m] < g.sentinel;
        const int tk = real ? ent[m] / g.slots : 0, j = real ? ent[m] - tk * g.slots : 0;
        wgt[m] = real && j < g.k ? g.wts[tk * g.k + j] : 1.0f;
      }
    }
    wait_vmem<0>();      // the epilogue's inputs have arrived (nothing else is queued)
    const int tn = t + per_x;
    wg_barrier();        // every wavefront is done reading this tile's buffers
    if (tn < t_end) {
      setup(tn);
      for (int s = 0; s < min(NS - 1, nst); ++s) issue(s, s);
    }

    // ---- epilogue.  Register q of acc[m][f] holds weight row
    // 8*(q/4) + 4*h + q%4 of fragment f for sorted row r32 of fragment m, so a
    // lane owns 16 outputs of one row: four runs of 4 consecutive columns.
    const int rbase = tile_row0 + wm * S::WROWS;
    if constexpr (GATEUP) {
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        const int row = rbase + m * 32 + r32;
#pragma unroll
        for (int f = 0; f < NF / 2; ++f) {
          // 32 neurons = one MX block of h, split over this lane and lane ^ 32
          const int n0 = tile_nt * (BN / 2) + wn * (S::WCOLS / 2) + 32 * f;
          float hv[16];
          float amax = 0.0f;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            hv[q] = swiglu(acc[m][f][q], acc[m][f + NF / 2][q]);
            amax = fmaxf(amax, fabsf(hv[q]));
          }
          amax = pair32_max(amax);
          const int e1 = mx_exponent(amax);
          const float inv1 = pow2_neg(e1), sc1 = pow2(e1);
          uint32_t whi[4];
          float rmax = 0.0f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            whi[r] = e4m3x4(hv[4 * r] * inv1, hv[4 * r + 1] * inv1, hv[4 * r + 2] * inv1,
                            hv[4 * r + 3] * inv1);
            // h - hi is exact in FP32
            const f32x2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(whi[r], 1.0f, false);
            const f32x2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(whi[r], 1.0f, true);
            hv[4 * r + 0] -= d0.x * sc1;
            hv[4 * r + 1] -= d0.y * sc1;
            hv[4 * r + 2] -= d1.x * sc1;
            hv[4 * r + 3] -= d1.y * sc1;
#pragma unroll
            for (int b = 0; b < 4; ++b) rmax = fmaxf(rmax, fabsf(hv[4 * r + b]));
          }
          rmax = pair32_max(rmax);
          const int e2 = mx_exponent(rmax);
          const float inv2 = pow2_neg(e2);
          uint8_t* q_hi = g.hq + (size_t)row * g.I + n0 + 4 * h;
          uint8_t* q_lo = q_hi + (size_t)g.cap * g.I;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            *reinterpret_cast<uint32_t*>(q_hi + 8 * r) = whi[r];
            *reinterpret_cast<uint32_t*>(q_lo + 8 * r) =
                e4m3x4(hv[4 * r] * inv2, hv[4 * r + 1] * inv2, hv[4 * r + 2] * inv2, hv[4 * r + 3] * inv2);
          }
          if (h == 0) {
            const size_t os = (size_t)row * (g.I >> 5) + (n0 >> 5);
            g.hs[os] = (uint8_t)(e1 + 127);
            g.hs[(size_t)g.cap * (g.I >> 5) + os] = (uint8_t)(e2 + 127);
          }
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        if (ent[m] < 0 || ent[m] >= g.sentinel) continue;
        uint16_t* out = g.out + (size_t)ent[m] * g.H;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int c0 = tile_nt * BN + wn * S::WCOLS + 32 * f + 4 * h;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (c0 + 8 * r < g.N) {
              // w * row, rounded once to BF16 (the slot buffer's format)
              const uint32_t b0 = f32_to_bf16_bits(__fmul_rn(acc[m][f][4 * r + 0], wgt[m]));
              const uint32_t b1 = f32_to_bf16_bits(__fmul_rn(acc[m][f][4 * r + 1], wgt[m]));
              const uint32_t b2 = f32_to_bf16_bits(__fmul_rn(acc[m][f][4 * r + 2], wgt[m]));
              const uint32_t b3 = f32_to_bf16_bits(__fmul_rn(acc[m][f][4 * r + 3], wgt[m]));
              *reinterpret_cast<uint2*>(out + c0 + 8 * r) = uint2{b0 | (b1 << 16), b2 | (b3 << 16)};
            }
          }
        }
      }
    }
    t = tn;
  }
}

// Tile shapes: BM is the align-sort block; BN weight rows per workgroup.
// Blocks of 32 / 64 rows stream their experts' weights (one M-block per
// expert at decode-like batches, HBM-bound); 128-row blocks take a 128 x 512
// tile in 64-K stages, the widest that three stages of LDS hold.
template <int BFMT, bool GATEUP>
hipError_t gemm_dispatch(const GemmArgs& a0, int bs, hipStream_t s) {
  GemmArgs a = a0;
  const int nx = a.nxcd;
  const int grid = std::max(nx, device_num_cus() / nx * nx);   // one workgroup per CU
#define MOE_GG(BM, BN, WM, WN, KS)                                                          \
  do {                                                                                      \
    a.n_ntiles = (GATEUP ? (a.N + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN);            \
    hipLaunchKernelGGL((grouped_gemm_kernel<BFMT, GATEUP, BM, BN, WM, WN, KS>), dim3(grid), \
                       dim3(64 * WM * WN), 0, s, a);                                        \
  } while (0)
  if (bs == 32) {
    // down with MX weights: 512 weight rows over eight wavefronts halve the
    // activation bytes (two terms) per weight byte; measured 5-10% faster
    // at 32-row blocks (Qwen3 B = 64: 48.9 -> 46.4 us; MXFP4: 125.6 ->
    // 113 us), while the FP8 128x128 layer was 5% slower (553 -> 582 us)
    if constexpr (!GATEUP && BFMT != W_FP8B128) {
      MOE_GG(32, 512, 1, 8, 2);
      return hipGetLastError();
    }
    // E2M1 weights: 256-K stages, so each weight row's slice of a stage is a
    // whole 128-byte line (128-K stages fetch half lines); measured on the
    // MXFP4 layer, outputs bit for bit the same: B = 128 314 -> 300 us,
    // B = 256 332 -> 311 us.  The down product gained nothing this way.
    if constexpr (GATEUP && BFMT == W_MXFP4) {
      if (a.K % 256 == 0) {
        MOE_GG(32, 256, 1, 4, 4);
        return hipGetLastError();
      }
    }
    MOE_GG(32, 256, 1, 4, 2);
  } else if (bs == 64) {
    MOE_GG(64, 256, 1, 4, 2);
  } else if constexpr (GATEUP) {
    MOE_GG(128, 256, 2, 2, 2);
  } else {
    // the down product reads two activation planes per weight row: eight
    // wavefronts keep more loads in flight from L2 (measured 13 -> 18 TB/s
    // for L2-resident streams) and interleave two waves per SIMD; gate_up's
    // 64 x 64 wave tiles would raise its LDS operand traffic instead
    MOE_GG(128, 256, 2, 4, 2);
  }
#undef MOE_GG
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gate_up(const moe_weights& W, const uint8_t* xq, const uint8_t* xs,
                                  int T, int slots, const int32_t* sorted,
                                  const int32_t* expert_ids, const int32_t* npp, int capacity,
                                  int bs, uint8_t* hq, uint8_t* hs, hipStream_t s) {
  if (capacity / bs == 0 || T == 0) return hipSuccess;
  // token row offsets are 32-bit in the kernel
  if ((long long)T * W.hidden >= (1ll << 32)) return hipErrorNotSupported;
  GemmArgs a{};
  a.a = xq;
  a.as = xs;
  a.sorted = sorted;
  a.slots = slots;
  a.sentinel = T * slots;
  a.b = reinterpret_cast<const uint8_t*>(W.w13);
  a.bs = W.w13_scale;
  a.expert_ids = expert_ids;
  a.npp = npp;
  a.hq = hq;
  a.hs = hs;
  a.cap = capacity;
  a.K = W.hidden;
  a.N = W.inter;
  a.I = W.inter;
  a.H = W.hidden;
  a.b_row_bytes = W.format == W_MXFP4 ? W.hidden / 2 : W.hidden;
  a.rows_per_expert = 2 * W.inter;
  a.nxcd = device_num_xcds();
  switch (W.format) {
    case W_MXFP8: return gemm_dispatch<W_MXFP8, true>(a, bs, s);
    case W_MXFP4: return gemm_dispatch<W_MXFP4, true>(a, bs, s);
    case W_FP8B128: return gemm_dispatch<W_FP8B128, true>(a, bs, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_grouped_down(const moe_weights& W, const uint8_t* hq, const uint8_t* hs,
                               const int32_t* sorted, const int32_t* expert_ids,
                               const int32_t* npp, int capacity, int bs, const float* wts, int T,
                               int k, uint16_t* slot_out, hipStream_t s) {
  if (capacity / bs == 0) return hipSuccess;
  GemmArgs a{};
  a.a = hq;
  a.as = hs;
  a.a_lo = hq + (size_t)capacity * W.inter;
  a.as_lo = hs + (size_t)capacity * (W.inter / 32);
  a.cap = capacity;
  a.b = reinterpret_cast<const uint8_t*>(W.w2);
  a.bs = W.w2_scale;
  a.expert_ids = expert_ids;
  a.npp = npp;
  a.sorted = sorted;
  a.wts = wts;
  a.out = slot_out;
  a.K = W.inter;
  a.N = W.hidden;
  a.I = W.inter;
  a.H = W.hidden;
  a.b_row_bytes = W.format == W_MXFP4 ? W.inter / 2 : W.inter;
  a.rows_per_expert = W.hidden;
  a.k = k;
  a.slots = k + W.num_shared;
  a.sentinel = T * a.slots;
  a.nxcd = device_num_xcds();
  switch (W.format) {
    case W_MXFP8: return gemm_dispatch<W_MXFP8, false>(a, bs, s);
    case W_MXFP4: return gemm_dispatch<W_MXFP4, false>(a, bs, s);
    case W_FP8B128: return gemm_dispatch<W_FP8B128, false>(a, bs, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace moe
