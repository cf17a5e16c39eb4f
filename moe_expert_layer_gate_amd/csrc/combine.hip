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
// one 64-lane pass over the row each: more rows in flight per CU, which the
// gather of scattered rows needs -- 4 waves per token took the Qwen3-shaped
// combine from 74 to 60 us) gather the token's (at most k) expert rows through
// the inverse map -- a gather, not a scatter-add, so no atomics and a
// deterministic result.  Each lane accumulates 8 columns at a time in fp32, in
// slot order, and rounds to bf16 once.  All accesses are 16 bytes wide.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// KMAX > 0: k <= KMAX, the slot loop is unrolled so that the (at most KMAX)
// row loads of a chunk are all in flight before the first is added; the sum
// is still formed in slot order.  KMAX == 0: any k, one slot at a time.
template <int KMAX>
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
  for (int c = part * kWave + lane; c < chunks; c += wpt * kWave) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    if constexpr (KMAX > 0) {
      uint4 v[KMAX];
#pragma unroll
      for (int s = 0; s < KMAX; ++s)
        if (rows[s] >= 0) v[s] = y_perm[static_cast<int64_t>(rows[s]) * chunks + c];
#pragma unroll
      for (int s = 0; s < KMAX; ++s) {
        if (rows[s] < 0) continue;  // uniform over the wave
        float f[8];
        unpack8(v[s], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += ws[s] * f[i];
      }
    } else {
      for (int s = 0; s < k; ++s) {
        const int r = __shfl(my_row, s);
        if (r < 0) continue;  // uniform over the wave
        const float w = __shfl(my_w, s);
        float f[8];
        unpack8(y_perm[static_cast<int64_t>(r) * chunks + c], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += w * f[i];
      }
    }
    if (shared_out) {
      float f[8];
      unpack8(shared_out[static_cast<int64_t>(t) * chunks + c], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    y[static_cast<int64_t>(t) * chunks + c] = o;
  }
}

}  // namespace

hipError_t launch_combine(const void* y_perm, const int32_t* token_slot_row, const float* topk_w,
                          const void* shared_out, int T, int k, int H, void* y, hipStream_t s) {
  auto kern = k <= 2 ? combine_kernel<2> : k <= 4 ? combine_kernel<4> : k <= 8 ? combine_kernel<8>
                                                                             : combine_kernel<0>;
  const int chunks = H / 8;
  const int per_row = ceil_div(chunks, kWave);          // 64-lane passes over one row
  const int want = ceil_div(65536, T);                  // waves per token for ~64k waves
  const int wpt = want < 1 ? 1 : (want < per_row ? want : per_row);
  const int64_t waves = static_cast<int64_t>(T) * wpt;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(ceil_div<int64_t>(waves, 4))), dim3(256), 0,
                     s, static_cast<const uint4*>(y_perm), token_slot_row, topk_w,
                     static_cast<const uint4*>(shared_out), T, k, chunks, wpt,
                     static_cast<uint4*>(y));
  return hipGetLastError();
}

}  // namespace moe
