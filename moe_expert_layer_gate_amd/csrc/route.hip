// Top-k softmax gate over router logits: one wavefront per token.
//
// Page "OverlapAdvisor: Modeling and Adapting Computation-Communication
// Overlap for Distributed MoE Serving", section 2.1: every token activates its
// top-k experts.  The weights are the softmax of the logits restricted to, and
// renormalised over, the k selected experts.
//
// Each lane holds ceil(E/64) logits of its token in registers as 64-bit keys
// (order-preserving image of the fp32 value in the high word, ~expert id in
// the low word), so one unsigned max picks the larger logit and, on a tie, the
// smaller expert id.  k rounds of a 6-step butterfly max over the wave select
// the experts in slot order; lane s keeps slot s.  The selection reads only
// the raw logits, so routing is bit-exact.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

__device__ __forceinline__ uint64_t logit_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0.0 and +0.0 are the same logit
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(0xFFFFFFFFu - static_cast<uint32_t>(e));
}

__device__ __forceinline__ float key_logit(uint64_t key) {
  uint32_t u = static_cast<uint32_t>(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

__device__ __forceinline__ int key_expert(uint64_t key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}

// One max step against lane permutation CTRL (a DPP control): every lane
// combines its key with the key of its partner lane.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL,
                                             0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)),
                                             CTRL, 0xF, 0xF, false);
  const uint64_t o = (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
  return o > v ? o : v;
}

// Max of a 64-bit key over the wave: within rows of 16 lanes by DPP (swap
// neighbours, swap pairs, mirror halves of 8, mirror the row), then across
// the four rows through two lane exchanges.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_u64<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_u64<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_u64<0x141>(v);  // row_half_mirror
  v = dpp_max_u64<0x140>(v);  // row_mirror
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off);
    uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const int lane = lane_id();
  const float* row = logits + static_cast<size_t>(t) * E;

  uint64_t key[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + kWave * j;
    key[j] = (e < E) ? logit_key(row[e], e) : 0ull;  // valid keys are > 0
  }

  uint64_t mine = 0;  // slot `lane` ends up here
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < VPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const int e = key_expert(best);
    if ((e & (kWave - 1)) == lane) {
#pragma unroll
      for (int j = 0; j < VPL; ++j)
        if (j == (e >> 6)) key[j] = 0ull;
    }
    if (lane == r) mine = best;
  }

  const float l0 = __shfl(key_logit(mine), 0);
  const float z = (lane < k) ? expf(key_logit(mine) - l0) : 0.0f;
  const float sum = wave_sum(z);
  if (lane < k) {
    topk_ids[static_cast<size_t>(t) * k + lane] = key_expert(mine);
    topk_w[static_cast<size_t>(t) * k + lane] = z / sum;
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k,
                             int32_t* ids, float* w, hipStream_t s) {
  const dim3 grid(ceil_div(T, 4)), block(256);
  const int vpl = ceil_div(E, kWave);
  if (vpl <= 1)
    hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 2)
    hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 4)
    hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 8)
    hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, ids, w);
  else
    hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
