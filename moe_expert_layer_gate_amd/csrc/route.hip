// Top-k softmax gate over router logits.
//
// Page "OverlapAdvisor: Modeling and Adapting Computation-Communication
// Overlap for Distributed MoE Serving", section 2.1: every token activates its
// top-k experts.  The weights are the softmax of the logits restricted to, and
// renormalised over, the k selected experts.
//
// Logits become 64-bit keys (order-preserving image of the fp32 value in the
// high word, ~expert id in the low word), so one unsigned max picks the larger
// logit and, on a tie, the smaller expert id; the selection reads only the raw
// logits, so routing is bit-exact.  k rounds each take the largest key left
// and remove it; slot s holds the key of round s.
//
// Up to 512 experts: one token per 16-lane row of a wave (four tokens per
// wave), each lane holding E/16 keys in registers.  A round is a max over the
// lane's keys and four DPP steps inside the row (no cross-row exchange, so no
// LDS-routed shuffles on the dependent chain), and the wave works on four
// tokens at once.  A row's loads are 16-byte pieces of its token's logits,
// 256 contiguous bytes per instruction.  Beyond 512 experts: one token per
// wave (keys E/64 per lane, the max over the whole wave).
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

// Max of a 64-bit key over each row of 16 lanes (DPP only).
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
  v = dpp_max_u64<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_u64<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_u64<0x141>(v);  // row_half_mirror
  v = dpp_max_u64<0x140>(v);  // row_mirror
  return v;
}

// Sum of a float over each row of 16 lanes, the same in every lane of the
// row (a butterfly: every lane adds its partners in the same order).
__device__ __forceinline__ float row_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1,
                                                              0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E,
                                                              0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141,
                                                              0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140,
                                                              0xF, 0xF, false));
  return v;
}

// One token per 16-lane row.  VPL keys per lane.  VEC: E % 4 == 0 and the
// lane loads float4 pieces -- key q = 4 j + c is expert 64 j + 4 lr + c --;
// otherwise key j is expert 16 j + lr.
template <int VPL, bool VEC>
__global__ __launch_bounds__(256) void route_topk_rows_kernel(
    const float* __restrict__ logits, int T, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int lr = threadIdx.x & 15;
  const bool live = t < T;   // dead rows run the same steps on zero keys
  const float* row = logits + static_cast<size_t>(live ? t : 0) * E;

  uint64_t key[VPL];
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < VPL / 4; ++j) {
      const int e0 = 64 * j + 4 * lr;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (live && e0 < E) v = *reinterpret_cast<const float4*>(row + e0);
      key[4 * j + 0] = (live && e0 + 0 < E) ? logit_key(v.x, e0 + 0) : 0ull;
      key[4 * j + 1] = (live && e0 + 1 < E) ? logit_key(v.y, e0 + 1) : 0ull;
      key[4 * j + 2] = (live && e0 + 2 < E) ? logit_key(v.z, e0 + 2) : 0ull;
      key[4 * j + 3] = (live && e0 + 3 < E) ? logit_key(v.w, e0 + 3) : 0ull;
    }
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = 16 * j + lr;
      key[j] = (live && e < E) ? logit_key(row[e], e) : 0ull;  // valid keys are > 0
    }
  }

  uint64_t mine0 = 0, mine1 = 0;  // slots lr and 16 + lr
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int q = 1; q < VPL; ++q) best = key[q] > best ? key[q] : best;
    best = row_max_u64(best);
    const int e = key_expert(best);
    const int owner = VEC ? (e >> 2) & 15 : e & 15;
    const int qe = VEC ? ((e >> 6) << 2) | (e & 3) : e >> 4;
    if (owner == lr) {
#pragma unroll
      for (int q = 0; q < VPL; ++q)
        if (q == qe) key[q] = 0ull;
    }
    if ((r & 15) == lr) {
      if (r < 16)
        mine0 = best;
      else
        mine1 = best;
    }
  }

  // weights: exp(l_s - l_0) / sum_j exp(l_j - l_0); l_0 is slot 0's logit
  const float l0 = key_logit(row_max_u64(lr == 0 ? mine0 : 0ull));
  const float z0 = (lr < k) ? expf(key_logit(mine0) - l0) : 0.0f;
  const float z1 = (16 + lr < k) ? expf(key_logit(mine1) - l0) : 0.0f;
  const float sum = row_sum(z0 + z1);
  if (live) {
    int32_t* ids = topk_ids + static_cast<size_t>(t) * k;
    float* wts = topk_w + static_cast<size_t>(t) * k;
    if (lr < k) {
      ids[lr] = key_expert(mine0);
      wts[lr] = z0 / sum;
    }
    if (16 + lr < k) {
      ids[16 + lr] = key_expert(mine1);
      wts[16 + lr] = z1 / sum;
    }
  }
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
  const dim3 block(256);
  if (E <= 512) {  // one token per 16-lane row
    const dim3 grid(ceil_div(T, 16));
    const int vpl = ceil_div(E, 16);
    if (E % 4 == 0) {
      if (vpl <= 4)
        hipLaunchKernelGGL((route_topk_rows_kernel<4, true>), grid, block, 0, s, logits, T, E, k, ids, w);
      else if (vpl <= 8)
        hipLaunchKernelGGL((route_topk_rows_kernel<8, true>), grid, block, 0, s, logits, T, E, k, ids, w);
      else if (vpl <= 16)
        hipLaunchKernelGGL((route_topk_rows_kernel<16, true>), grid, block, 0, s, logits, T, E, k, ids, w);
      else
        hipLaunchKernelGGL((route_topk_rows_kernel<32, true>), grid, block, 0, s, logits, T, E, k, ids, w);
    } else {
      if (vpl <= 1)
        hipLaunchKernelGGL((route_topk_rows_kernel<1, false>), grid, block, 0, s, logits, T, E, k, ids, w);
      else if (vpl <= 4)
        hipLaunchKernelGGL((route_topk_rows_kernel<4, false>), grid, block, 0, s, logits, T, E, k, ids, w);
      else if (vpl <= 8)
        hipLaunchKernelGGL((route_topk_rows_kernel<8, false>), grid, block, 0, s, logits, T, E, k, ids, w);
      else if (vpl <= 16)
        hipLaunchKernelGGL((route_topk_rows_kernel<16, false>), grid, block, 0, s, logits, T, E, k, ids, w);
      else
        hipLaunchKernelGGL((route_topk_rows_kernel<32, false>), grid, block, 0, s, logits, T, E, k, ids, w);
    }
    return hipGetLastError();
  }
  // one token per wave
  const dim3 grid(ceil_div(T, 4));
  const int vpl = ceil_div(E, kWave);
  if (vpl <= 16)
    hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
