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
// wave), each lane holding E/16 keys in registers, sorted once.  A round is
// four DPP max steps over the lanes' first keys inside the row (no cross-row
// exchange, so no LDS-routed shuffles on the dependent chain), and the wave
// works on four tokens at once.  A row's loads are 16-byte pieces of its
// token's logits, 256 contiguous bytes per instruction.  Beyond 512 experts:
// one token per wave (keys E/64 per lane, the max over the whole wave).
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

// ---------------------------------------------------------------------------
// Up to 512 experts: one token per 16-lane row.
//
// Keys as doubles.  The selection order -- larger logit first, equal logits
// by smaller expert id, -0.0 equal to +0.0 -- is that of the 42-bit integer
// (ordered image of the fp32 logit) << 10 | (1023 - e); placed in the
// mantissa of a double with exponent 0 (a value in [1, 2)), it orders the
// same way as that double, and no key is a zero, a denormal, an infinity or
// a NaN.  So one v_max_f64 / v_min_f64 compares two keys (instead of a 64-bit
// integer compare and two selects); they are issued as written, without the
// NaN-quieting the compiler would otherwise put in front of them.  Keys are
// unique.  Each lane sorts its keys once (Batcher's odd-even merge network, a
// max and a min per comparator); a round takes the row's largest head by four
// DPP steps, and the lane that held it drops its head (one shift of its list).
// ---------------------------------------------------------------------------
constexpr uint32_t kKeyHi = 0x3FF00000u;   // exponent of [1, 2)

__device__ __forceinline__ double route_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;                                  // -0.0 -> +0.0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);                 // ordered image
  const uint32_t hi = kKeyHi | (u >> 22);
  const uint32_t lo = (u << 10) | static_cast<uint32_t>(1023 - e);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

__device__ __forceinline__ int route_key_expert(double d) {
  return 1023 - static_cast<int>(static_cast<uint32_t>(__double_as_longlong(d)) & 1023u);
}

__device__ __forceinline__ float route_key_logit(double d) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(d));
  uint32_t u = static_cast<uint32_t>(b >> 10);                    // 32 bits of order
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

__device__ __forceinline__ double max_f64(double a, double b) {
  double r;
  asm volatile("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ double min_f64(double a, double b) {
  double r;
  asm volatile("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Largest key over each row of 16 lanes (DPP only).
template <int CTRL>
__device__ __forceinline__ double dpp_max_f64(double v) {
  // every lane's source lane is inside its row, so no old value is needed
  const long long u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(u), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(u >> 32), CTRL, 0xF, 0xF, true);
  const double o = __longlong_as_double((static_cast<long long>(hi) << 32) |
                                        static_cast<uint32_t>(lo));
  return max_f64(v, o);
}

__device__ __forceinline__ double row_max_f64(double v) {
  v = dpp_max_f64<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_f64<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_f64<0x141>(v);  // row_half_mirror
  v = dpp_max_f64<0x140>(v);  // row_mirror
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

// Sort N keys descending in registers: Batcher's odd-even merge sort, every
// index a compile-time constant once the loops unroll.
template <int N>
__device__ __forceinline__ void sort_desc(double (&a)[N]) {
#pragma unroll
  for (int p = 1; p < N; p <<= 1)
#pragma unroll
    for (int k = p; k >= 1; k >>= 1)
#pragma unroll
      for (int j = k % p; j + k < N; j += 2 * k)
#pragma unroll
        for (int i = 0; i < k; ++i)
          if (i + j + k < N && (i + j) / (2 * p) == (i + j + k) / (2 * p)) {
            const double x = a[i + j], y = a[i + j + k];
            a[i + j] = max_f64(x, y);
            a[i + j + k] = min_f64(x, y);
          }
}

// The L largest of N keys, sorted descending, in a[0..L): for L = N / 2 the
// two halves are sorted, the larger of a[i] and a[N-1-i] forms a bitonic
// sequence holding the top half, and a bitonic network sorts it; otherwise a
// full sort.
template <int N, int L>
__device__ __forceinline__ void top_desc(double (&a)[N]) {
  if constexpr (L * 2 == N && N >= 4) {
    double lo[N / 2], hi[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      lo[i] = a[i];
      hi[i] = a[N / 2 + i];
    }
    sort_desc<N / 2>(lo);
    sort_desc<N / 2>(hi);
#pragma unroll
    for (int i = 0; i < N / 2; ++i) a[i] = max_f64(lo[i], hi[N / 2 - 1 - i]);
    // a[0..N/2) descends then ascends: bitonic merge into descending order
#pragma unroll
    for (int d = N / 4; d >= 1; d >>= 1)
#pragma unroll
      for (int i = 0; i < N / 2; ++i)
        if ((i & d) == 0) {
          const double x = a[i], y = a[i + d];
          a[i] = max_f64(x, y);
          a[i + d] = min_f64(x, y);
        }
  } else {
    sort_desc<N>(a);
  }
}

// One token per 16-lane row; VPL keys per lane, of which the first L (sorted)
// can ever be taken (L = min(VPL, the largest k this instance serves)).
// VEC: E % 4 == 0 and the lane loads float4 pieces -- key q = 4 j + c is
// expert 64 j + 4 lr + c --; otherwise key j is expert 16 j + lr.  FULL: E is
// exactly 16 VPL, so no key is padding.
template <int VPL, int L, bool VEC, bool FULL>
__global__ __launch_bounds__(256) void route_topk_rows_kernel(
    const float* __restrict__ logits, int T, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int lr = threadIdx.x & 15;
  const bool live = t < T;   // rows past T run on the last token and store nothing
  const float* row = logits + static_cast<size_t>(live ? t : T - 1) * E;
  const double kNone = __longlong_as_double(0);   // +0.0: below every key

  double key[VPL];
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < VPL / 4; ++j) {
      const int e0 = 64 * j + 4 * lr;
      const bool in = FULL || e0 < E;
      // the row's first piece stands in for pieces past E (never used)
      const float4 v = *reinterpret_cast<const float4*>(row + (in ? e0 : 0));
      key[4 * j + 0] = route_key(v.x, e0 + 0);
      key[4 * j + 1] = route_key(v.y, e0 + 1);
      key[4 * j + 2] = route_key(v.z, e0 + 2);
      key[4 * j + 3] = route_key(v.w, e0 + 3);
      if (!FULL && !in)
#pragma unroll
        for (int c = 0; c < 4; ++c) key[4 * j + c] = kNone;
    }
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = 16 * j + lr;
      const bool in = FULL || e < E;
      key[j] = route_key(row[in ? e : 0], e);
      if (!FULL && !in) key[j] = kNone;
    }
  }
  top_desc<VPL, L>(key);

  double mine0 = kNone, mine1 = kNone;  // slots lr and 16 + lr
  for (int r = 0; r < k; ++r) {
    const double best = row_max_f64(key[0]);
    if (key[0] == best) {  // the one lane of the row that held it
#pragma unroll
      for (int q = 0; q + 1 < L; ++q) key[q] = key[q + 1];
      key[L - 1] = kNone;
    }
    if ((r & 15) == lr) {
      if (r < 16)
        mine0 = best;
      else
        mine1 = best;
    }
  }

  // weights: exp(l_s - l_0) / sum_j exp(l_j - l_0); l_0 is slot 0's logit
  const float l0 = route_key_logit(row_max_f64(lr == 0 ? mine0 : kNone));
  const float z0 = (lr < k) ? expf(route_key_logit(mine0) - l0) : 0.0f;
  const float z1 = (16 + lr < k) ? expf(route_key_logit(mine1) - l0) : 0.0f;
  const float sum = row_sum(z0 + z1);
  if (live) {
    int32_t* ids = topk_ids + static_cast<size_t>(t) * k;
    float* wts = topk_w + static_cast<size_t>(t) * k;
    // (only non-finite logits could decode to an id past E)
    if (lr < k) {
      ids[lr] = min(route_key_expert(mine0), E - 1);
      wts[lr] = z0 / sum;
    }
    if (16 + lr < k) {
      ids[16 + lr] = min(route_key_expert(mine1), E - 1);
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

template <int VPL, bool VEC, bool FULL>
void launch_rows_l(dim3 grid, const float* logits, int T, int E, int k, int32_t* ids, float* w,
                   hipStream_t s) {
  // a lane can give at most min(k, VPL) of the token's k experts: keep that
  // many of its sorted keys
  constexpr int L8 = VPL < 8 ? VPL : 8, L16 = VPL < 16 ? VPL : 16, L32 = VPL < 32 ? VPL : 32;
  if (k <= 8)
    hipLaunchKernelGGL((route_topk_rows_kernel<VPL, L8, VEC, FULL>), grid, dim3(256), 0, s,
                       logits, T, E, k, ids, w);
  else if (k <= 16)
    hipLaunchKernelGGL((route_topk_rows_kernel<VPL, L16, VEC, FULL>), grid, dim3(256), 0, s,
                       logits, T, E, k, ids, w);
  else
    hipLaunchKernelGGL((route_topk_rows_kernel<VPL, L32, VEC, FULL>), grid, dim3(256), 0, s,
                       logits, T, E, k, ids, w);
}

template <int VPL, bool VEC>
void launch_rows(dim3 grid, const float* logits, int T, int E, int k, int32_t* ids, float* w,
                 hipStream_t s) {
  if (E == 16 * VPL)
    launch_rows_l<VPL, VEC, true>(grid, logits, T, E, k, ids, w, s);
  else
    launch_rows_l<VPL, VEC, false>(grid, logits, T, E, k, ids, w, s);
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k,
                             int32_t* ids, float* w, hipStream_t s) {
  if (E <= 512) {  // one token per 16-lane row
    const dim3 grid(ceil_div(T, 16));
    const int vpl = ceil_div(E, 16);
    if (E % 4 == 0) {
      if (vpl <= 4) launch_rows<4, true>(grid, logits, T, E, k, ids, w, s);
      else if (vpl <= 8) launch_rows<8, true>(grid, logits, T, E, k, ids, w, s);
      else if (vpl <= 16) launch_rows<16, true>(grid, logits, T, E, k, ids, w, s);
      else launch_rows<32, true>(grid, logits, T, E, k, ids, w, s);
    } else {
      if (vpl <= 1) launch_rows<1, false>(grid, logits, T, E, k, ids, w, s);
      else if (vpl <= 4) launch_rows<4, false>(grid, logits, T, E, k, ids, w, s);
      else if (vpl <= 8) launch_rows<8, false>(grid, logits, T, E, k, ids, w, s);
      else if (vpl <= 16) launch_rows<16, false>(grid, logits, T, E, k, ids, w, s);
      else launch_rows<32, false>(grid, logits, T, E, k, ids, w, s);
    }
    return hipGetLastError();
  }
  // one token per wave
  const dim3 grid(ceil_div(T, 4));
  hipLaunchKernelGGL(route_topk_kernel<16>, grid, dim3(256), 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
