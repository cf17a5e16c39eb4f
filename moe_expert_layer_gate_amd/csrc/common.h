// Shared device-side definitions of the HIP library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Pack two floats into two bf16 (lo in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_bits(lo)) |
         (static_cast<uint32_t>(f32_to_bf16_bits(hi)) << 16);
}

// E4M3FN code of v (already scaled), round to nearest even, saturated to
// +-448.  The clamp keeps every input inside the finite range before the
// hardware conversion, so no NaN code can appear.
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
  const float m = 448.0f;
  a = fminf(fmaxf(a, -m), m);
  b = fminf(fmaxf(b, -m), m);
  c = fminf(fmaxf(c, -m), m);
  d = fminf(fmaxf(d, -m), m);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return static_cast<uint32_t>(r);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Exclusive scan of one value per thread over a block of up to 1024 threads.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total_out) {
  __shared__ int warp_sums[16];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) warp_sums[w] = incl;
  __syncthreads();
  int base = 0, total = 0;
  const int nw = blockDim.x >> 6;
  for (int i = 0; i < nw; ++i) {
    if (i < w) base += warp_sums[i];
    total += warp_sums[i];
  }
  __syncthreads();
  *total_out = total;
  return base + incl - v;
}

template <typename T>
__host__ __device__ __forceinline__ T ceil_div(T a, T b) { return (a + b - 1) / b; }

// Owner of entry u of a table whose experts hold consecutive runs starting at
// s_start[0..E_L) (non-decreasing; u below the total): the last expert whose
// run starts at or before u, which is never an empty one.
__device__ __forceinline__ int run_owner(const int* s_start, int E_L, int u) {
  int lo = 0, hi = E_L - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_start[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// m-tile table of the GEMM paths that run one block per tile (skinny,
// pipelined, MX), built by one block whose thread e < E_L owns local expert e
// with cnt rows; every thread of the block calls it.  Entries [start, start +
// tiles) of expert e hold {e, start, tiles, 0} and *n_tiles the total; the
// block's threads write the entries together.  sync (fused decode FFN; may be
// null): sync[0], the ticket counter, and sync[1 + i], the up tiles finished
// for m-tile i, start at 0.  status (may be null): the FFN's flag word,
// cleared for the launch that follows.
__device__ __forceinline__ void build_tile_table(int e, int E_L, int cnt, int tile_m,
                                                 int4* __restrict__ info, int32_t* __restrict__ n_tiles,
                                                 int32_t* __restrict__ sync,
                                                 int32_t* __restrict__ status) {
  __shared__ int s_start[1024];
  const int tiles = e < E_L ? ceil_div(cnt, tile_m) : 0;
  int total;
  const int start = block_exclusive_scan(tiles, &total);
  if (e < E_L) s_start[e] = start;
  __syncthreads();
  for (int u = threadIdx.x; u < total; u += blockDim.x) {
    const int o = run_owner(s_start, E_L, u);
    const int first = s_start[o];
    const int n = (o + 1 < E_L ? s_start[o + 1] : total) - first;
    info[u] = make_int4(o, first, n, 0);
    if (sync) sync[1 + u] = 0;
  }
  if (threadIdx.x == 0) {
    *n_tiles = total;
    if (sync) sync[0] = 0;
    if (status) *status = 0;
  }
}

}  // namespace moe
