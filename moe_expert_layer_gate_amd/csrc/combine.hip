// Combine: gate-weighted sum of a token's expert outputs back in token order.
//
// Page "CascadeEP: Asynchronous Expert Execution for MoE Prefill under
// Attention Imbalance", Appendix C, "Output return and combine": every routed
// contribution is weighted by its routing coefficient exactly once, the
// contributions are summed at the token's origin, and the shared-expert output
// is added.  Page "OverlapAdvisor ...", section 4.2.1: unpermute restores the
// token order.
//
// wpt wavefronts per token, as many as give the chip about 64 k waves (up to
// one pass over the row each: more rows in flight per CU, which the gather of
// scattered rows needs -- 4 waves per token took the Qwen3-shaped combine from
// 74 to 60 us) gather the token's (at most k) expert rows through the inverse
// map -- a gather, not a scatter-add, so no atomics and a deterministic
// result.  A pass reads 2 or 4 KB contiguous from every slot row (each lane
// 2 or 4 pieces of 8 columns, 1 KB apart), fewer, longer runs per row than
// 1 KB passes: 8 % (DeepSeek-V3-shaped shard) and 13 % (Qwen3 shape) faster.
// Each lane accumulates in fp32, in slot order, and rounds to bf16 once.
// All accesses are 16 bytes wide and
// non-temporal: every y_perm (and shared-expert) row is read once and y is
// written once, and the streaming hint took the DeepSeek-V3-shaped shard's
// combine from 293 to about 250 us (y_perm loads 12 %, y stores 3 %).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream(uint4 o, uint4* p) {
  const u32x4 v = {o.x, o.y, o.z, o.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// A pass of a wave covers U x 64 chunks of the row: lane l takes chunks c0 +
// u * 64 (u < U) of every slot row, so each row is read U kilobytes at a time
// in one contiguous run.  KMAX > 0: k <= KMAX, the slot loop is unrolled so
// that all the (at most KMAX x U) row loads of a pass are in flight before the
// first is added; the sum is still formed in slot order.  KMAX == 0: any k,
// one slot at a time.
template <int KMAX, int U>
__global__ __launch_bounds__(256) void combine_kernel(
    const uint4* __restrict__ y_perm, const int32_t* __restrict__ token_slot_row,
    const float* __restrict__ topk_w, const uint4* __restrict__ shared_out, int T, int k,
    int chunks, int wpt, uint4* __restrict__ y) {
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = gw / wpt, part = gw - t * wpt;
  if (t >= T) return;
  const int lane = lane_id();
  // Slot rows and weights of this token: lane s < k holds slot s.
  int my_row = -1;
  float my_w = 0.0f;
  if (lane < k) {
    my_row = token_slot_row[static_cast<int64_t>(t) * k + lane];
    my_w = topk_w[static_cast<int64_t>(t) * k + lane];
  }
  int rows[KMAX > 0 ? KMAX : 1];
  float ws[KMAX > 0 ? KMAX : 1];
  if constexpr (KMAX > 0) {
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      rows[s] = s < k ? __shfl(my_row, s) : -1;
      ws[s] = __shfl(my_w, s);
    }
  }
  for (int c0 = part * U * kWave + lane; c0 - lane < chunks; c0 += wpt * U * kWave) {
    bool in[U];
#pragma unroll
    for (int u = 0; u < U; ++u) in[u] = c0 + u * kWave < chunks;
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
    if constexpr (KMAX > 0) {
      uint4 v[KMAX][U];
#pragma unroll
      for (int s = 0; s < KMAX; ++s)
        if (rows[s] >= 0)
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (in[u]) v[s][u] = load_stream(y_perm + static_cast<int64_t>(rows[s]) * chunks + c0 +
                                             u * kWave);
#pragma unroll
      for (int s = 0; s < KMAX; ++s) {
        if (rows[s] < 0) continue;  // uniform over the wave
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (!in[u]) continue;
          float f[8];
          unpack8(v[s][u], f);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[u][i] += ws[s] * f[i];
        }
      }
    } else {
      for (int s = 0; s < k; ++s) {
        const int r = __shfl(my_row, s);
        if (r < 0) continue;  // uniform over the wave
        const float w = __shfl(my_w, s);
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (in[u]) v[u] = load_stream(y_perm + static_cast<int64_t>(r) * chunks + c0 + u * kWave);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (!in[u]) continue;
          float f[8];
          unpack8(v[u], f);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[u][i] += w * f[i];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!in[u]) continue;
      const int c = c0 + u * kWave;
      if (shared_out) {
        float f[8];
        unpack8(load_stream(shared_out + static_cast<int64_t>(t) * chunks + c), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] += f[i];
      }
      uint4 o;
      o.x = pack_bf16x2(acc[u][0], acc[u][1]);
      o.y = pack_bf16x2(acc[u][2], acc[u][3]);
      o.z = pack_bf16x2(acc[u][4], acc[u][5]);
      o.w = pack_bf16x2(acc[u][6], acc[u][7]);
      store_stream(o, y + static_cast<int64_t>(t) * chunks + c);
    }
  }
}

template <int U>
void launch_combine_u(const void* y_perm, const int32_t* token_slot_row, const float* topk_w,
                      const void* shared_out, int T, int k, int chunks, void* y, hipStream_t s) {
  auto kern = k <= 2 ? combine_kernel<2, U> : k <= 4 ? combine_kernel<4, U>
            : k <= 8 ? combine_kernel<8, U> : combine_kernel<0, U>;
  const int per_row = ceil_div(chunks, U * kWave);      // passes over one row
  const int want = ceil_div(65536, T);                  // waves per token for ~64k waves
  const int wpt = want < 1 ? 1 : (want < per_row ? want : per_row);
  const int64_t waves = static_cast<int64_t>(T) * wpt;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(ceil_div<int64_t>(waves, 4))), dim3(256), 0,
                     s, static_cast<const uint4*>(y_perm), token_slot_row, topk_w,
                     static_cast<const uint4*>(shared_out), T, k, chunks, wpt,
                     static_cast<uint4*>(y));
}

}  // namespace

// 4 KB runs of every row when a row has more than one of them (DeepSeek-V3-
// shaped rows of 14 KB: 258 -> 237 us for the EP8 shard), else 2 KB (rows of
// 4 KB, Qwen3 shape: 56.6 -> 49.1 us; 4 KB runs left half the waves and took
// 51.6 us).
hipError_t launch_combine(const void* y_perm, const int32_t* token_slot_row, const float* topk_w,
                          const void* shared_out, int T, int k, int H, void* y, hipStream_t s) {
  const int chunks = H / 8;
  if (chunks > 4 * kWave)
    launch_combine_u<4>(y_perm, token_slot_row, topk_w, shared_out, T, k, chunks, y, s);
  else
    launch_combine_u<2>(y_perm, token_slot_row, topk_w, shared_out, T, k, chunks, y, s);
  return hipGetLastError();
}

}  // namespace moe
