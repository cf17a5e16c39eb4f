// Top-k softmax gate over router logits.
//
// Page "OverlapAdvisor: Modeling and Adapting Computation-Communication
// Overlap for Distributed MoE Serving", section 2.1: every token activates its
// top-k experts.  The weights are the softmax of the logits restricted to, and
// renormalised over, the k selected experts.
//
// Logits become 64-bit keys (order-preserving image of the fp32 value above
// the complement of the expert id), so one max picks the larger logit and, on
// a tie, the smaller expert id; the selection reads only the raw logits, so
// routing is bit-exact.  Slot s holds the key of rank s.
//
// Up to 512 experts: one token per row of 8 lanes (up to 256 experts) or 16
// lanes, each lane holding E/8 or E/16 keys in registers.  Each lane sorts
// the largest of its keys once; then every lane merges its sorted list with a
// partner lane's, taken by DPP, keeping the largest (log2 of the row width
// levels, no cross-row exchange and no LDS).  The wave works on 8 or 4 tokens
// at once, with no data-dependent loop.  A row's loads are 16-byte pieces of
// its token's logits, 128 or 256 contiguous bytes per instruction.  Beyond 512
// experts: one token per wave (keys E/64 per lane), k rounds of a wave max
// that each take the largest key left and remove it.
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
// Up to 512 experts: one token per row of R lanes (R = 8 for up to 256
// experts, else 16), 64 / R tokens per wave.
//
// Keys as doubles.  The selection order -- larger logit first, equal logits
// by smaller expert id, -0.0 equal to +0.0 -- is that of the 42-bit integer
// (ordered image of the fp32 logit) << 10 | (1023 - e); placed in the
// mantissa of a double with exponent 0 (a value in [1, 2)), it orders the
// same way as that double, and no key is a zero, a denormal, an infinity or
// a NaN.  So one v_max_f64 / v_min_f64 compares two keys (instead of a 64-bit
// integer compare and two selects); they are issued as written, without the
// NaN-quieting the compiler would otherwise put in front of them.  Keys are
// unique, so every sorted list of the largest keys of a set is unique too.
//
// Each lane keeps the LK largest of its keys, sorted (LK = 8, 16 or 32, the
// smallest power of two >= k), by Batcher's odd-even merge sort on groups
// and the largest-half merge below.  Then log2(R) merge levels: a lane takes
// its partner lane's list by DPP (partners xor 1, xor 2, mirror of 8, mirror
// of 16: after each level the lanes of a group of 2, 4, 8, 16 hold the same
// list) and keeps the LK largest of both lists.  After the last level every
// lane of the row holds the token's LK largest keys in slot order; lane l
// takes slots l, l + R, ... .  No step depends on a value from another row.
// ---------------------------------------------------------------------------
constexpr uint32_t kKeyHi = 0x3FF00000u;   // exponent of [1, 2)

// Ordered 32-bit image of an fp32 logit: the unsigned order of images is the
// order of the logits, and -0.0 and +0.0 share one image.  Non-negative x with
// bits u maps to u + 2^31, negative x with magnitude bits m to 2^31 - m.
__device__ __forceinline__ uint32_t logit_order(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t s = static_cast<uint32_t>(static_cast<int32_t>(u) >> 31);   // ~0 if negative
  return (u ^ (s | 0x80000000u)) - s;
}

// id_bits = 1023 - e (10 bits).
__device__ __forceinline__ double route_key(float v, uint32_t id_bits) {
  const uint32_t o = logit_order(v);
  const uint32_t hi = __builtin_amdgcn_alignbit(kKeyHi >> 10, o, 22);   // kKeyHi | o >> 22
  const uint32_t lo = (o << 10) | id_bits;
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

__device__ __forceinline__ int route_key_expert(double d) {
  return 1023 - static_cast<int>(static_cast<uint32_t>(__double_as_longlong(d)) & 1023u);
}

__device__ __forceinline__ float route_key_logit(double d) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(d));
  const uint32_t o = static_cast<uint32_t>(b >> 10);               // the ordered image
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : (0u - o));
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

// The partner lane's value under DPP control CTRL (the partner is in the
// same row of 16, so no old value is needed).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(u), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(u >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<uint32_t>(lo));
}

// Partners of the merge levels: xor 1, xor 2, mirror inside 8, mirror inside 16.
template <int LEVEL>
constexpr int kLevelCtrl = LEVEL == 0 ? 0xB1 : LEVEL == 1 ? 0x4E : LEVEL == 2 ? 0x141 : 0x140;

// Sum of a float over each row of R lanes, the same in every lane of the row
// (a butterfly over the merge levels' partners).
template <int R>
__device__ __forceinline__ float row_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              kLevelCtrl<0>, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              kLevelCtrl<1>, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              kLevelCtrl<2>, 0xF, 0xF, false));
  if constexpr (R == 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                kLevelCtrl<3>, 0xF, 0xF, false));
  return v;
}

// Compare-exchange: the larger key to position i, the smaller to j.
template <int N>
__device__ __forceinline__ void cex(double (&a)[N], int i, int j) {
  const double x = a[i], y = a[j];
  a[i] = max_f64(x, y);
  a[j] = min_f64(x, y);
}

// Sort a[0..N) descending: Batcher's odd-even merge sort, every index a
// compile-time constant once the loops unroll.
template <int N, int CAP>
__device__ __forceinline__ void sort_desc(double (&a)[CAP]) {
#pragma unroll
  for (int p = 1; p < N; p <<= 1)
#pragma unroll
    for (int k = p; k >= 1; k >>= 1)
#pragma unroll
      for (int j = k % p; j + k < N; j += 2 * k)
#pragma unroll
        for (int i = 0; i < k; ++i)
          if (i + j + k < N && (i + j) / (2 * p) == (i + j + k) / (2 * p)) cex(a, i + j, i + j + k);
}

// Bitonic merge: a[0..M) descends then ascends -> a[0..M) descending.
template <int M, int CAP>
__device__ __forceinline__ void bitonic_desc(double (&a)[CAP]) {
#pragma unroll
  for (int d = M / 2; d >= 1; d >>= 1)
#pragma unroll
    for (int i = 0; i < M; ++i)
      if ((i & d) == 0) cex(a, i, i + d);
}

// The L largest of N keys (N, L powers of two), sorted descending, in
// a[0..L): each half reduced to its L largest, then the larger of a[i] and
// b[L-1-i] (the L largest of both, a bitonic sequence) merged.
template <int N, int L>
__device__ __forceinline__ void top_sorted(double (&a)[N]) {
  if constexpr (N <= L) {
    sort_desc<N>(a);
  } else {
    double lo[N / 2], hi[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      lo[i] = a[i];
      hi[i] = a[N / 2 + i];
    }
    top_sorted<N / 2, L>(lo);
    top_sorted<N / 2, L>(hi);
#pragma unroll
    for (int i = 0; i < L; ++i) a[i] = max_f64(lo[i], hi[L - 1 - i]);
    bitonic_desc<L>(a);
  }
}

// One merge level: this lane's sorted list a[0..N) and the partner's become
// the min(2N, LK) largest keys of both, sorted, in a.
template <int LEVEL, int N, int LK>
__device__ __forceinline__ void merge_level(double (&a)[LK]) {
  double b[N];
#pragma unroll
  for (int i = 0; i < N; ++i) b[i] = dpp_f64<kLevelCtrl<LEVEL>>(a[i]);
  if constexpr (2 * N <= LK) {   // both lists whole: descending ++ ascending
#pragma unroll
    for (int i = 0; i < N; ++i) a[N + i] = b[N - 1 - i];
    bitonic_desc<2 * N>(a);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) a[i] = max_f64(a[i], b[N - 1 - i]);
    bitonic_desc<N>(a);
  }
}

constexpr int cmin(int a, int b) { return a < b ? a : b; }

// a[idx] for a lane-dependent idx in [0, M): a selection tree on idx's bits
// (levels whose bit is a constant after unrolling fold away).
template <int M>
__device__ __forceinline__ double pick(const double (&a)[M], int idx) {
  double t[M];
#pragma unroll
  for (int i = 0; i < M; ++i) t[i] = a[i];
#pragma unroll
  for (int w = M / 2, bit = 1; w >= 1; w >>= 1, bit <<= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = (idx & bit) ? t[2 * i + 1] : t[2 * i];
  return t[0];
}

// One token per row of R lanes; VPL keys per lane; LK (8, 16 or 32, >= k)
// keys kept.  VEC: E % 4 == 0 and the lane loads float4 pieces -- key q =
// 4 j + c is expert 4 R j + 4 lr + c --; otherwise key j is expert R j + lr.
// FULL: E is exactly R VPL, so no key is padding.
template <int R, int VPL, int LK, bool VEC, bool FULL>
__global__ __launch_bounds__(256) void route_topk_rows_kernel(
    const float* __restrict__ logits, int T, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
  static_assert(R == 8 || R == 16, "rows of 8 or 16 lanes");
  constexpr int kLog = R == 16 ? 4 : 3;
  const int t = blockIdx.x * (256 / R) + (threadIdx.x >> kLog);
  const int lr = threadIdx.x & (R - 1);
  const bool live = t < T;   // rows past T run on the last token and store nothing
  const float* row = logits + static_cast<size_t>(live ? t : T - 1) * E;
  const double kNone = __longlong_as_double(0);   // +0.0: below every key

  double key[VPL];
  if constexpr (VEC) {
    // 1023 - e = 1023 - 4 R j - 4 lr - c splits into disjoint bit fields:
    // 3 - c (bits 0-1), 4 (R - 1 - lr) (bits 2 .. log2(4R) - 1) and
    // 1024 - 4 R (j + 1) (above), so ORs assemble it
    const uint32_t lane_bits = static_cast<uint32_t>(4 * (R - 1 - lr));
#pragma unroll
    for (int j = 0; j < VPL / 4; ++j) {
      const int e0 = 4 * R * j + 4 * lr;
      const bool in = FULL || e0 < E;
      // the row's first piece stands in for pieces past E (never used)
      const float4 v = *reinterpret_cast<const float4*>(row + (in ? e0 : 0));
      const uint32_t jb = static_cast<uint32_t>(1024 - 4 * R * (j + 1)) | lane_bits;
      key[4 * j + 0] = route_key(v.x, jb | 3u);
      key[4 * j + 1] = route_key(v.y, jb | 2u);
      key[4 * j + 2] = route_key(v.z, jb | 1u);
      key[4 * j + 3] = route_key(v.w, jb);
      if (!FULL && !in)
#pragma unroll
        for (int c = 0; c < 4; ++c) key[4 * j + c] = kNone;
    }
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = R * j + lr;
      const bool in = FULL || e < E;
      key[j] = route_key(row[in ? e : 0], static_cast<uint32_t>(1023 - e));
      if (!FULL && !in) key[j] = kNone;
    }
  }

  // the lane's N0 largest keys, sorted, then the merge levels
  constexpr int N0 = cmin(VPL, LK);
  top_sorted<VPL, N0>(key);
  double a[LK];
#pragma unroll
  for (int i = 0; i < LK; ++i) a[i] = i < N0 ? key[i] : kNone;
  constexpr int N1 = cmin(2 * N0, LK), N2 = cmin(2 * N1, LK), N3 = cmin(2 * N2, LK);
  merge_level<0, N0, LK>(a);
  merge_level<1, N1, LK>(a);
  merge_level<2, N2, LK>(a);
  if constexpr (R == 16) merge_level<3, N3, LK>(a);

  // lane lr: slots lr, lr + R, ...; weights exp(l_s - l_0) / sum_j exp(l_j - l_0)
  constexpr int SPL = LK > R ? LK / R : 1;
  const float l0 = route_key_logit(a[0]);
  float z[SPL];
  int id[SPL];
  float zsum = 0.0f;
#pragma unroll
  for (int q = 0; q < SPL; ++q) {
    const int s = q * R + lr;
    const double m = pick<LK>(a, LK > R ? s : (lr & (LK - 1)));
    z[q] = s < k ? expf(route_key_logit(m) - l0) : 0.0f;
    // (only non-finite logits could decode to an id past E)
    id[q] = min(route_key_expert(m), E - 1);
    zsum += z[q];
  }
  const float sum = row_sum<R>(zsum);
  if (live) {
    int32_t* ids = topk_ids + static_cast<size_t>(t) * k;
    float* wts = topk_w + static_cast<size_t>(t) * k;
#pragma unroll
    for (int q = 0; q < SPL; ++q) {
      const int s = q * R + lr;
      if (s < k) {
        ids[s] = id[q];
        wts[s] = z[q] / sum;
      }
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

// Rows of 8 lanes up to this many experts (at most 32 keys per lane), rows
// of 16 above it.
constexpr int kRows8MaxE = 256;

template <int R, int VPL, bool VEC, bool FULL>
void launch_rows_l(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                   hipStream_t s) {
  const dim3 grid(ceil_div(T, 256 / R));
  if (k <= 8)
    hipLaunchKernelGGL((route_topk_rows_kernel<R, VPL, 8, VEC, FULL>), grid, dim3(256), 0, s,
                       logits, T, E, k, ids, w);
  else if (k <= 16)
    hipLaunchKernelGGL((route_topk_rows_kernel<R, VPL, 16, VEC, FULL>), grid, dim3(256), 0, s,
                       logits, T, E, k, ids, w);
  else
    hipLaunchKernelGGL((route_topk_rows_kernel<R, VPL, 32, VEC, FULL>), grid, dim3(256), 0, s,
                       logits, T, E, k, ids, w);
}

template <int R, int VPL, bool VEC>
void launch_rows(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                 hipStream_t s) {
  if (E == R * VPL)
    launch_rows_l<R, VPL, VEC, true>(logits, T, E, k, ids, w, s);
  else
    launch_rows_l<R, VPL, VEC, false>(logits, T, E, k, ids, w, s);
}

template <int R>
void launch_rows_r(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                   hipStream_t s) {
  const int vpl = ceil_div(E, R);
  if (E % 4 == 0) {
    if (vpl <= 4) launch_rows<R, 4, true>(logits, T, E, k, ids, w, s);
    else if (vpl <= 8) launch_rows<R, 8, true>(logits, T, E, k, ids, w, s);
    else if (vpl <= 16) launch_rows<R, 16, true>(logits, T, E, k, ids, w, s);
    else launch_rows<R, 32, true>(logits, T, E, k, ids, w, s);
  } else {
    if (vpl <= 1) launch_rows<R, 1, false>(logits, T, E, k, ids, w, s);
    else if (vpl <= 4) launch_rows<R, 4, false>(logits, T, E, k, ids, w, s);
    else if (vpl <= 8) launch_rows<R, 8, false>(logits, T, E, k, ids, w, s);
    else if (vpl <= 16) launch_rows<R, 16, false>(logits, T, E, k, ids, w, s);
    else launch_rows<R, 32, false>(logits, T, E, k, ids, w, s);
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k,
                             int32_t* ids, float* w, hipStream_t s) {
  if (E <= kRows8MaxE) {
    launch_rows_r<8>(logits, T, E, k, ids, w, s);
    return hipGetLastError();
  }
  if (E <= 512) {
    launch_rows_r<16>(logits, T, E, k, ids, w, s);
    return hipGetLastError();
  }
  // one token per wave
  const dim3 grid(ceil_div(T, 4));
  hipLaunchKernelGGL(route_topk_kernel<16>, grid, dim3(256), 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
