// Dispatch: the expert-major permutation of the local (token, slot) pairs and
// the gather of their activation rows.
//
// Page "CascadeEP: Asynchronous Expert Execution for MoE Prefill under
// Attention Imbalance", Appendix C, "Grouped FFN invocations": per-expert row
// offsets from the selected token counts, rows grouped contiguously by expert,
// activations packed with their quantisation metadata, and an inverse map from
// each row to its token and routing slot.  Page "OverlapAdvisor ...", section
// 4.2.1: permute groups tokens by expert.
//
// The permutation is a stable counting sort done in three launches (two while
// the histogram below is small enough for every scatter block to read it: the
// scatter blocks then do the scan themselves), with no float and no
// order-dependent atomics (the result is deterministic):
//   1. count:   each block of 256 tokens builds, in LDS, one 256-bit mask per
//               local expert (bit i = token i of the block picked it) and
//               writes the popcounts as its per-expert histogram;
//   2. scan:    one block turns the [blocks x E_L] histogram into per-block
//               bases (exclusive scan over blocks) and the expert offsets
//               (exclusive scan over experts);
//   3. scatter: each block rebuilds its masks; a pair's rank inside its block
//               is the popcount of the mask bits below its token, so rows come
//               out in token order inside every expert segment.
// A slot that repeats an expert already picked by an earlier slot of the
// same token is skipped, which keeps every (token, expert) at most once and so
// every position in range whatever ids the caller passes.
// Up to 256 tokens (decode batches) the three steps run in one block and one
// launch.
//
// Masked (fixed-capacity) layout, cap > 0 (page "ExpertPlex": masked grouped-
// GEMM layout; page "OverlapAdvisor ...", Table 7: low-latency dispatch feeds
// the GroupGEMM with no permute step): expert e's rows start at e * cap instead
// of at the scan of the counts; everything else is the same sort, so a row's
// rank inside its expert, and hence every per-row result, is the same in both
// layouts.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kTokBlock = 256;  // tokens per count/scatter block
constexpr int kMaskWords = kTokBlock / 32;

// Local expert of every slot of token t (slots s < k), -1 where the expert
// is not local or repeats one of an earlier slot.  KMAX >= k is a compile-time
// bound, so the slots live in registers (fully unrolled, no indexed arrays).
template <int KMAX>
__device__ __forceinline__ void token_local_experts(const int32_t* __restrict__ topk_ids, int t,
                                                    int k, int e_lo, int E_L, int* le) {
  int ids[KMAX];
#pragma unroll
  for (int s = 0; s < KMAX; ++s) ids[s] = s < k ? topk_ids[static_cast<size_t>(t) * k + s] : -1;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    bool rep = false;
#pragma unroll
    for (int q = 0; q < s; ++q) rep |= ids[q] == ids[s];
    const int e = ids[s] - e_lo;
    le[s] = (s < k && !rep && e >= 0 && e < E_L) ? e : -1;
  }
}

// Build the per-expert token masks of block b in LDS from the local experts
// of this thread's token (t < T).
template <int KMAX>
__device__ __forceinline__ void build_masks(uint32_t* mask, const int* le, bool has_token,
                                            int E_L) {
  for (int i = threadIdx.x; i < E_L * kMaskWords; i += blockDim.x) mask[i] = 0u;
  __syncthreads();
  if (has_token) {
#pragma unroll
    for (int s = 0; s < KMAX; ++s)
      if (le[s] >= 0)
        atomicOr(&mask[le[s] * kMaskWords + (threadIdx.x >> 5)], 1u << (threadIdx.x & 31));
  }
  __syncthreads();
}

template <int KMAX>
__global__ __launch_bounds__(kTokBlock) void index_count_kernel(
    const int32_t* __restrict__ topk_ids, int T, int k, int e_lo, int E_L,
    int32_t* __restrict__ blk_hist) {
  extern __shared__ uint32_t mask[];
  const int t = blockIdx.x * kTokBlock + threadIdx.x;
  int le[KMAX];
  if (t < T) token_local_experts<KMAX>(topk_ids, t, k, e_lo, E_L, le);
  build_masks<KMAX>(mask, le, t < T, E_L);
  for (int e = threadIdx.x; e < E_L; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) c += __popc(mask[e * kMaskWords + w]);
    blk_hist[static_cast<size_t>(blockIdx.x) * E_L + e] = c;
  }
}

__global__ __launch_bounds__(1024) void index_scan_kernel(
    const int32_t* __restrict__ blk_hist, int nblk, int E_L, int cap,
    int32_t* __restrict__ blk_base, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets) {
  // E_L <= 1024 = blockDim.x.  Thread (part, e) owns expert e over the part's
  // run of blocks; the parts' sums are scanned in LDS, then every part writes
  // its bases.  Part 0 of expert e is thread e.
  __shared__ int part_sum[1024];
  const int parts = 1024 / E_L;
  const int e = threadIdx.x % E_L, part = threadIdx.x / E_L;
  const int chunk = ceil_div(nblk, parts);
  const int b0 = part * chunk, b1 = min(nblk, b0 + chunk);
  const bool mine = part < parts;
  int sum = 0;
  if (mine)
    for (int b = b0; b < b1; ++b) sum += blk_hist[static_cast<size_t>(b) * E_L + e];
  part_sum[threadIdx.x] = mine ? sum : 0;
  __syncthreads();
  int base = 0, run = 0;
  if (mine) {
    for (int q = 0; q < parts; ++q) {
      const int v = part_sum[q * E_L + e];
      if (q < part) base += v;
      run += v;
    }
    int acc = base;
    for (int b = b0; b < b1; ++b) {
      blk_base[static_cast<size_t>(b) * E_L + e] = acc;
      acc += blk_hist[static_cast<size_t>(b) * E_L + e];
    }
  }
  int total;
  const bool first_part = static_cast<int>(threadIdx.x) < E_L;  // part 0: one thread per expert
  const int off = block_exclusive_scan(first_part ? run : 0, &total);
  if (first_part) {
    counts[e] = run;
    offsets[e] = cap ? e * cap : off;
  }
  if (threadIdx.x == 0) offsets[E_L] = cap ? E_L * cap : total;
}

// Rank of token slot t (bit t % 256 of the block) among the block's tokens
// that picked the expert whose mask starts at m.
__device__ __forceinline__ int mask_rank(const uint32_t* m, int tb) {
  const int wi = tb >> 5;
  int rank = __popc(m[wi] & ((1u << (tb & 31)) - 1u));
  for (int w = 0; w < wi; ++w) rank += __popc(m[w]);
  return rank;
}

// Count, scan and scatter of at most 256 tokens in one block of 1024 threads
// (thread e < E_L owns expert e in the scan; thread t < T owns token t).
// With tile_m > 0 the block also writes the m-tile table of the GEMMs that
// read these segments (build_tile_table).  mask: E_L * (kMaskWords + 1)
// words of LDS.
template <int KMAX>
__device__ __forceinline__ void index_small_block(
    const int32_t* __restrict__ topk_ids, int T, int k, int e_lo, int E_L, int cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_slot,
    int32_t* __restrict__ token_slot_row, uint32_t* mask, int tile_m, int4* __restrict__ info,
    int32_t* __restrict__ n_tiles, int32_t* __restrict__ sync, int32_t* __restrict__ status) {
  int* s_off = reinterpret_cast<int*>(mask + E_L * kMaskWords);
  int le[KMAX];
  if (static_cast<int>(threadIdx.x) < T) token_local_experts<KMAX>(topk_ids, threadIdx.x, k, e_lo, E_L, le);
  build_masks<KMAX>(mask, le, static_cast<int>(threadIdx.x) < T, E_L);
  const int e = threadIdx.x;
  int c = 0;
  if (e < E_L)
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) c += __popc(mask[e * kMaskWords + w]);
  int total;
  const int off = block_exclusive_scan(c, &total);
  if (e < E_L) {
    const int o = cap ? e * cap : off;
    counts[e] = c;
    offsets[e] = o;
    s_off[e] = o;
  }
  if (e == 0) offsets[E_L] = cap ? E_L * cap : total;
  if (tile_m > 0) build_tile_table(e, E_L, c, tile_m, info, n_tiles, sync, status);
  __syncthreads();
  const int t = threadIdx.x;
  if (t >= T) return;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    if (s < k) {
      int pos = -1;
      if (le[s] >= 0) {
        pos = s_off[le[s]] + mask_rank(mask + le[s] * kMaskWords, t);
        row_token[pos] = t;
        row_slot[pos] = s;
      }
      token_slot_row[static_cast<size_t>(t) * k + s] = pos;
    }
  }
}

template <int KMAX>
__global__ __launch_bounds__(1024) void index_small_kernel(
    const int32_t* __restrict__ topk_ids, int T, int k, int e_lo, int E_L, int cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_slot,
    int32_t* __restrict__ token_slot_row) {
  extern __shared__ uint32_t mask[];
  index_small_block<KMAX>(topk_ids, T, k, e_lo, E_L, cap, counts, offsets, row_token, row_slot,
                          token_slot_row, mask, 0, nullptr, nullptr, nullptr, nullptr);
}

template <int KMAX>
__global__ __launch_bounds__(kTokBlock) void index_scatter_kernel(
    const int32_t* __restrict__ topk_ids, int T, int k, int e_lo, int E_L,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_slot,
    int32_t* __restrict__ token_slot_row) {
  extern __shared__ uint32_t mask[];
  const int t = blockIdx.x * kTokBlock + threadIdx.x;
  int le[KMAX];
  if (t < T) token_local_experts<KMAX>(topk_ids, t, k, e_lo, E_L, le);
  build_masks<KMAX>(mask, le, t < T, E_L);
  if (t >= T) return;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    if (s < k) {
      const int e = le[s];
      int pos = -1;
      if (e >= 0) {
        pos = offsets[e] + blk_base[static_cast<size_t>(blockIdx.x) * E_L + e] +
              mask_rank(mask + e * kMaskWords, threadIdx.x);
        row_token[pos] = t;
        row_slot[pos] = s;
      }
      token_slot_row[static_cast<size_t>(t) * k + s] = pos;
    }
  }
}

// The scan folded into the scatter while nblk x (the histogram's nblk x E_L
// entries) is at most kFoldReads: every block reads the whole histogram and
// derives what it needs -- the experts' offsets and, per expert, the count of
// its pairs in earlier blocks -- then scatters its tokens like
// index_scatter_kernel (block b's tokens are threads 0..255); block 0 also
// writes counts and offsets.
// Thread (part, e) of the 1024 sums expert e over the part's run of blocks,
// as index_scan_kernel does.  mask: E_L * (kMaskWords + 1) words of LDS.
constexpr int64_t kFoldReads = 1 << 22;   // 16 MB of histogram reads in all

template <int KMAX>
__global__ __launch_bounds__(1024) void index_scan_scatter_kernel(
    const int32_t* __restrict__ topk_ids, int T, int k, int e_lo, int E_L, int cap,
    const int32_t* __restrict__ blk_hist, int nblk, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
    int32_t* __restrict__ row_slot, int32_t* __restrict__ token_slot_row) {
  extern __shared__ uint32_t mask[];
  int* s_base = reinterpret_cast<int*>(mask + E_L * kMaskWords);
  __shared__ int part_all[1024], part_before[1024];
  const int b = blockIdx.x;
  const int parts = 1024 / E_L;
  const int e = threadIdx.x % E_L, part = threadIdx.x / E_L;
  const int chunk = ceil_div(nblk, parts);
  const int b0 = part * chunk, b1 = min(nblk, b0 + chunk);
  int all = 0, before = 0;
  if (part < parts)
    for (int bb = b0; bb < b1; ++bb) {
      const int v = blk_hist[static_cast<size_t>(bb) * E_L + e];
      all += v;
      before += bb < b ? v : 0;
    }
  part_all[threadIdx.x] = part < parts ? all : 0;
  part_before[threadIdx.x] = part < parts ? before : 0;
  __syncthreads();
  const bool first_part = static_cast<int>(threadIdx.x) < E_L;  // thread e owns expert e
  int total_e = 0, before_e = 0;
  if (first_part)
    for (int q = 0; q < parts; ++q) {
      total_e += part_all[q * E_L + e];
      before_e += part_before[q * E_L + e];
    }
  int total;
  const int off = block_exclusive_scan(first_part ? total_e : 0, &total);
  if (first_part) {
    const int o = cap ? e * cap : off;
    s_base[e] = o + before_e;
    if (b == 0) {
      counts[e] = total_e;
      offsets[e] = o;
    }
  }
  if (b == 0 && threadIdx.x == 0) offsets[E_L] = cap ? E_L * cap : total;
  // this block's tokens
  const int tb = static_cast<int>(threadIdx.x);
  const int t = b * kTokBlock + tb;
  const bool has_token = tb < kTokBlock && t < T;
  int le[KMAX];
  if (has_token) token_local_experts<KMAX>(topk_ids, t, k, e_lo, E_L, le);
  build_masks<KMAX>(mask, le, has_token, E_L);
  if (!has_token) return;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    if (s < k) {
      const int x = le[s];
      int pos = -1;
      if (x >= 0) {
        pos = s_base[x] + mask_rank(mask + x * kMaskWords, tb);
        row_token[pos] = t;
        row_slot[pos] = s;
      }
      token_slot_row[static_cast<size_t>(t) * k + s] = pos;
    }
  }
}

// Whether row j of a masked layout (cap > 0) holds a pair: the first
// counts[e] rows of expert e's block [e cap, (e + 1) cap) do.
__device__ __forceinline__ bool masked_row_used(const int32_t* counts, int cap, int j) {
  if (!cap) return true;
  const int e = j / cap;
  return j - e * cap < counts[e];
}

// Row gather of bf16 activations: dst[j] = src[rows[j]] for j < *n_rows
// (rows == nullptr: identity), skipping unused rows of a masked layout.  One
// wavefront per row, 16-byte accesses.
__global__ __launch_bounds__(256) void gather_rows_bf16_kernel(
    const uint4* __restrict__ src, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ n_rows, int n_rows_host, int chunks_per_row,
    const int32_t* __restrict__ counts, int cap, uint4* __restrict__ dst) {
  const int n = n_rows ? *n_rows : n_rows_host;
  const int wpb = blockDim.x >> 6;
  for (int j = blockIdx.x * wpb + (threadIdx.x >> 6); j < n; j += gridDim.x * wpb) {
    if (!masked_row_used(counts, cap, j)) continue;  // uniform over the wave
    const int r = rows ? rows[j] : j;
    const uint4* s = src + static_cast<size_t>(r) * chunks_per_row;
    uint4* d = dst + static_cast<size_t>(j) * chunks_per_row;
    for (int c = lane_id(); c < chunks_per_row; c += kWave) d[c] = s[c];
  }
}

// The same gather into panel layout [H/32][panel_rows][32].  A work item is
// 16 consecutive destination rows x 8 panels; lane l of the wavefront moves
// the 16 bytes l % 4 of row l / 4 in each panel, so every store instruction
// writes one contiguous kilobyte (16 rows of a panel) and the source rows
// are read in 64-byte runs.
__global__ __launch_bounds__(256) void gather_rows_panel_kernel(
    const uint4* __restrict__ src, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ n_rows, int n_rows_host, int chunks_per_row,
    int64_t panel_rows, const int32_t* __restrict__ counts, int cap, uint4* __restrict__ dst) {
  constexpr int kPanelsPerItem = 8;
  const int n = n_rows ? *n_rows : n_rows_host;
  const int wpb = blockDim.x >> 6;
  const int lane = lane_id(), sub = lane & 3;
  const int panels = chunks_per_row >> 2;
  const int pblocks = (panels + kPanelsPerItem - 1) / kPanelsPerItem;
  const int64_t items = static_cast<int64_t>((n + 15) >> 4) * pblocks;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * wpb + (threadIdx.x >> 6); it < items;
       it += static_cast<int64_t>(gridDim.x) * wpb) {
    const int grp = static_cast<int>(it / pblocks);
    const int p0 = static_cast<int>(it - static_cast<int64_t>(grp) * pblocks) * kPanelsPerItem;
    const int j = grp * 16 + (lane >> 2);
    if (j >= n || !masked_row_used(counts, cap, j)) continue;
    const int r = rows ? rows[j] : j;
    const uint4* s = src + static_cast<size_t>(r) * chunks_per_row + sub;
    uint4* d = dst + static_cast<size_t>(j) * 4 + sub;
    if (p0 + kPanelsPerItem <= panels) {
      uint4 v[kPanelsPerItem];
#pragma unroll
      for (int u = 0; u < kPanelsPerItem; ++u) v[u] = s[(p0 + u) * 4];
#pragma unroll
      for (int u = 0; u < kPanelsPerItem; ++u) d[(p0 + u) * panel_rows * 4] = v[u];
    } else {
      for (int p = p0; p < panels; ++p) d[p * panel_rows * 4] = s[p * 4];
    }
  }
}

// Panel packing, [batch][rows][cols] -> [batch][cols/32][rows][32] (bf16).
// Threads walk the destination in order (16 bytes each), so writes are
// contiguous and each group of four threads reads one 64-byte run.
__global__ __launch_bounds__(256) void pack_panel_kernel(const uint4* __restrict__ src,
                                                         int64_t batch, int64_t rows,
                                                         int64_t cols, uint4* __restrict__ dst) {
  const int64_t units = cols / 8;               // 16-byte units per row
  const int64_t per_mat = rows * units;
  const int64_t total = batch * per_mat;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < total;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t b = u / per_mat, v = u - b * per_mat;
    const int64_t panel = v / (rows * 4), w = v - panel * rows * 4;
    const int64_t r = w >> 2, sub = w & 3;
    dst[u] = src[b * per_mat + r * units + panel * 4 + sub];
  }
}

// Panel packing of MX weight scales, [batch][rows][cols/128] dwords (four
// E8M0 bytes: one 128-element K step of a row) -> [batch][cols/128][rows].
// Threads walk the destination in order, so writes are contiguous.
__global__ __launch_bounds__(256) void pack_scales_mx_kernel(const uint32_t* __restrict__ src,
                                                             int64_t batch, int64_t rows,
                                                             int64_t steps,
                                                             uint32_t* __restrict__ dst) {
  const int64_t per_mat = rows * steps;
  const int64_t total = batch * per_mat;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < total;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t b = u / per_mat, v = u - b * per_mat;
    const int64_t k = v / rows, r = v - k * rows;
    dst[u] = src[b * per_mat + r * steps + k];
  }
}

// Row gather with per-128 group E4M3 quantisation: scale = amax/448 (1 for an
// all-zero group), code = RNE(v / scale) (IEEE fp32 division) saturated.
// A group of 128 bf16 is 16 lanes x 8 values; a wave covers 4 groups per step.
// `parts` waves share a row, each taking every parts-th 64-lane pass of it (a
// few rows -- a decode batch -- would otherwise run their passes one after
// another in one wave each).
// Wave gw of nwaves.
__device__ __forceinline__ void quant_rows_fp8(
    int gw, int nwaves, const uint4* __restrict__ src, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ n_rows, int n_rows_host, int H, int parts,
    const int32_t* __restrict__ counts, int cap,
    uint2* __restrict__ dst, float* __restrict__ dst_scale) {
  const int n = n_rows ? *n_rows : n_rows_host;
  const int chunks = H >> 3;  // 8 bf16 per chunk
  const int groups = H >> 7;
  const int lane = lane_id();
  const int part = gw % parts, slot = gw / parts, slots = nwaves / parts;
  if (slot >= slots) return;  // uniform over the wave
  for (int j = slot; j < n; j += slots) {
    if (!masked_row_used(counts, cap, j)) continue;  // uniform over the wave
    const int r = rows ? rows[j] : j;
    const uint4* s = src + static_cast<size_t>(r) * chunks;
    uint2* d = dst + static_cast<size_t>(j) * chunks;
    // chunks is a multiple of 16, so the 16 lanes of a group are all active or
    // all idle in every step, and the xor-shuffles below stay inside a group.
    for (int c = part * kWave + lane; c < chunks; c += kWave * parts) {
      const uint4 v = s[c];
      float f[8];
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(wv[i] << 16);
        f[2 * i + 1] = __uint_as_float(wv[i] & 0xFFFF0000u);
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
      const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
      uint2 q;
      q.x = f32x4_to_e4m3x4(f[0] / sc, f[1] / sc, f[2] / sc, f[3] / sc);
      q.y = f32x4_to_e4m3x4(f[4] / sc, f[5] / sc, f[6] / sc, f[7] / sc);
      d[c] = q;
      if ((lane & 15) == 0) dst_scale[static_cast<size_t>(j) * groups + (c >> 4)] = sc;
    }
  }
}

// 128 x 128 block quantisation of bf16 matrices (weights at load time).
// One block of 256 threads per 128 x 128 tile; partial row tiles allowed.
__global__ __launch_bounds__(256) void quant_blocks_kernel(
    const uint16_t* __restrict__ src, int64_t rows, int64_t cols,
    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int64_t mat = blockIdx.z;
  const int64_t rb = blockIdx.y, cb = blockIdx.x;
  const int64_t nrb = (rows + 127) / 128, ncb = cols / 128;
  const uint16_t* s = src + mat * rows * cols;
  uint8_t* q = codes + mat * rows * cols;
  // Thread i handles row (i >> 1) of the tile, columns (i & 1) * 64 .. +64.
  const int64_t r = rb * 128 + (threadIdx.x >> 1);
  const int64_t c0 = cb * 128 + (threadIdx.x & 1) * 64;
  const bool valid = r < rows;
  float f[64];
  float amax = 0.0f;
  if (valid) {
    const uint4* p = reinterpret_cast<const uint4*>(s + r * cols + c0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 v = p[i];
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[8 * i + 2 * j] = __uint_as_float(wv[j] << 16);
        f[8 * i + 2 * j + 1] = __uint_as_float(wv[j] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  __shared__ float wmax[4];
  if (lane_id() == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (threadIdx.x == 0) scales[mat * nrb * ncb + rb * ncb + cb] = sc;
  if (valid) {
    uint4* d = reinterpret_cast<uint4*>(q + r * cols + c0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 o;
      o.x = f32x4_to_e4m3x4(f[16 * i + 0] / sc, f[16 * i + 1] / sc, f[16 * i + 2] / sc, f[16 * i + 3] / sc);
      o.y = f32x4_to_e4m3x4(f[16 * i + 4] / sc, f[16 * i + 5] / sc, f[16 * i + 6] / sc, f[16 * i + 7] / sc);
      o.z = f32x4_to_e4m3x4(f[16 * i + 8] / sc, f[16 * i + 9] / sc, f[16 * i + 10] / sc, f[16 * i + 11] / sc);
      o.w = f32x4_to_e4m3x4(f[16 * i + 12] / sc, f[16 * i + 13] / sc, f[16 * i + 14] / sc, f[16 * i + 15] / sc);
      d[i] = o;
    }
  }
}

// ---------------------------------------------------------------------------
// MX formats (OCP MX): blocks of 32 consecutive elements of a row share one
// E8M0 scale 2^(c - 127), c = floor(log2 amax) - emax + 127 clamped to
// [0, 254] (an all-zero block takes c = 0); elements are the element
// format's round-to-nearest-even of v / 2^(c - 127), saturated.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int mx_code(float amax, int emax) {
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff);
  if (e == 0) return 0;  // zero or subnormal: at or below 2^-127
  const int s = e - 127 - emax;
  return (s < -127 ? -127 : s) + 127;
}

// E2M1 code of v (already divided by the block scale): nearest of 0, 0.5, 1,
// 1.5, 2, 3, 4, 6, a tie going to the even mantissa bit, beyond 6 saturated.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return c | (__float_as_uint(v) >> 31 << 3);
}

// MXFP4 conversion of bf16 rows (weights at load time): one thread per block
// of 32 elements; codes two per byte, low nibble first.
__global__ __launch_bounds__(256) void quant_mx4_kernel(const uint4* __restrict__ src,
                                                        int64_t blocks, uint4* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; b < blocks;
       b += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float f[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[b * 4 + i];
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[8 * i + 2 * j] = __uint_as_float(wv[j] << 16);
        f[8 * i + 2 * j + 1] = __uint_as_float(wv[j] & 0xFFFF0000u);
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
    const int c = mx_code(amax, 2);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i / 8] |= e2m1_code(ldexpf(f[i], 127 - c)) << (4 * (i % 8));
    codes[b] = make_uint4(w[0], w[1], w[2], w[3]);
    scales[b] = static_cast<uint8_t>(c);
  }
}

// Row gather with MXFP8 packing: dst[j] = E4M3 codes of src[rows[j]] with one
// E8M0 scale per 32 elements (rows == nullptr: identity); masked-layout rows
// that hold no pair are skipped.  `parts` wavefronts per row (as in the
// block-FP8 gather); four lanes (8 elements each) make a block.
// Wave gw of nwaves.
__device__ __forceinline__ void quant_rows_mx8(
    int gw, int nwaves, const uint4* __restrict__ src, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ n_rows, int n_rows_host, int H, int parts,
    const int32_t* __restrict__ counts, int cap,
    uint2* __restrict__ dst, uint8_t* __restrict__ dst_scale) {
  const int n = n_rows ? *n_rows : n_rows_host;
  const int chunks = H >> 3;
  const int lane = lane_id();
  const int part = gw % parts, slot = gw / parts, slots = nwaves / parts;
  if (slot >= slots) return;  // uniform over the wave
  for (int j = slot; j < n; j += slots) {
    if (!masked_row_used(counts, cap, j)) continue;  // uniform over the wave
    const int r = rows ? rows[j] : j;
    const uint4* s = src + static_cast<size_t>(r) * chunks;
    uint2* d = dst + static_cast<size_t>(j) * chunks;
    // chunks is a multiple of 16, so the four lanes of a block are all active
    for (int c = part * kWave + lane; c < chunks; c += kWave * parts) {
      const uint4 v = s[c];
      float f[8];
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(wv[i] << 16);
        f[2 * i + 1] = __uint_as_float(wv[i] & 0xFFFF0000u);
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      const int code = mx_code(amax, 8);
      const int sh = 127 - code;
      uint2 q;
      q.x = f32x4_to_e4m3x4(ldexpf(f[0], sh), ldexpf(f[1], sh), ldexpf(f[2], sh), ldexpf(f[3], sh));
      q.y = f32x4_to_e4m3x4(ldexpf(f[4], sh), ldexpf(f[5], sh), ldexpf(f[6], sh), ldexpf(f[7], sh));
      d[c] = q;
      if ((lane & 3) == 0) dst_scale[static_cast<size_t>(j) * (H >> 5) + (c >> 2)] = code;
    }
  }
}

__global__ __launch_bounds__(256) void gather_rows_fp8_kernel(
    const uint4* __restrict__ src, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ n_rows, int n_rows_host, int H, int parts,
    const int32_t* __restrict__ counts, int cap,
    uint2* __restrict__ dst, float* __restrict__ dst_scale) {
  const int wpb = blockDim.x >> 6;
  quant_rows_fp8(blockIdx.x * wpb + (threadIdx.x >> 6), gridDim.x * wpb, src, rows, n_rows,
                 n_rows_host, H, parts, counts, cap, dst, dst_scale);
}

__global__ __launch_bounds__(256) void gather_rows_mx8_kernel(
    const uint4* __restrict__ src, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ n_rows, int n_rows_host, int H, int parts,
    const int32_t* __restrict__ counts, int cap,
    uint2* __restrict__ dst, uint8_t* __restrict__ dst_scale) {
  const int wpb = blockDim.x >> 6;
  quant_rows_mx8(blockIdx.x * wpb + (threadIdx.x >> 6), gridDim.x * wpb, src, rows, n_rows,
                 n_rows_host, H, parts, counts, cap, dst, dst_scale);
}

// The layer's front for at most 256 tokens in one launch: block 0 builds the
// index and the m-tile table (index_small_block); the other blocks quantise
// the T token rows of x (QK 1: block-FP8, 2: MXFP8; QK 0: none, one block),
// `parts` waves per row.  The two parts share no data.
template <int KMAX, int QK>
__global__ __launch_bounds__(1024) void index_front_kernel(
    const int32_t* __restrict__ topk_ids, int T, int k, int e_lo, int E_L, int cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_slot,
    int32_t* __restrict__ token_slot_row, int tile_m, int4* __restrict__ info,
    int32_t* __restrict__ n_tiles, int32_t* __restrict__ sync, int32_t* __restrict__ status,
    const uint4* __restrict__ x, int H, int parts, uint2* __restrict__ xq, void* xq_scale) {
  extern __shared__ uint32_t mask[];
  if (blockIdx.x == 0) {
    index_small_block<KMAX>(topk_ids, T, k, e_lo, E_L, cap, counts, offsets, row_token, row_slot,
                            token_slot_row, mask, tile_m, info, n_tiles, sync, status);
    return;
  }
  if constexpr (QK != 0) {
    const int wpb = blockDim.x >> 6;
    const int gw = (blockIdx.x - 1) * wpb + (threadIdx.x >> 6);
    const int nw = (gridDim.x - 1) * wpb;
    if constexpr (QK == 1)
      quant_rows_fp8(gw, nw, x, nullptr, nullptr, T, H, parts, nullptr, 0, xq,
                     static_cast<float*>(xq_scale));
    else
      quant_rows_mx8(gw, nw, x, nullptr, nullptr, T, H, parts, nullptr, 0, xq,
                     static_cast<uint8_t*>(xq_scale));
  }
}

}  // namespace

size_t index_scratch_bytes(int T, int E_L) {
  const size_t nblk = static_cast<size_t>(ceil_div(T, kTokBlock));
  return 2 * nblk * static_cast<size_t>(E_L) * sizeof(int32_t);
}

hipError_t launch_index_build(const int32_t* topk_ids, int T, int k, int e_lo, int E_L, int cap,
                              int32_t* counts, int32_t* offsets, int32_t* row_token,
                              int32_t* row_slot, int32_t* token_slot_row,
                              void* scratch, hipStream_t s) {
  if (T <= kTokBlock) {
    const size_t lds = static_cast<size_t>(E_L) * (kMaskWords + 1) * sizeof(uint32_t);
    hipLaunchKernelGGL(k <= 8 ? index_small_kernel<8> : index_small_kernel<32>, dim3(1), dim3(1024),
                       lds, s, topk_ids, T, k, e_lo, E_L, cap, counts, offsets, row_token,
                       row_slot, token_slot_row);
    return hipGetLastError();
  }
  const int nblk = ceil_div(T, kTokBlock);
  int32_t* blk_hist = static_cast<int32_t*>(scratch);
  int32_t* blk_base = blk_hist + static_cast<size_t>(nblk) * E_L;
  const size_t lds = static_cast<size_t>(E_L) * kMaskWords * sizeof(uint32_t);
  hipLaunchKernelGGL(k <= 8 ? index_count_kernel<8> : index_count_kernel<32>, dim3(nblk),
                     dim3(kTokBlock), lds, s,
                     topk_ids, T, k, e_lo, E_L, blk_hist);
  if (static_cast<int64_t>(nblk) * nblk * E_L <= kFoldReads) {  // two launches
    const size_t lds2 = static_cast<size_t>(E_L) * (kMaskWords + 1) * sizeof(uint32_t);
    hipLaunchKernelGGL(k <= 8 ? index_scan_scatter_kernel<8> : index_scan_scatter_kernel<32>,
                       dim3(nblk), dim3(1024), lds2, s, topk_ids, T, k, e_lo, E_L, cap, blk_hist,
                       nblk, counts, offsets, row_token, row_slot, token_slot_row);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(index_scan_kernel, dim3(1), dim3(1024), 0, s,
                     blk_hist, nblk, E_L, cap, blk_base, counts, offsets);
  hipLaunchKernelGGL(k <= 8 ? index_scatter_kernel<8> : index_scatter_kernel<32>, dim3(nblk),
                     dim3(kTokBlock), lds, s,
                     topk_ids, T, k, e_lo, E_L, blk_base, offsets, row_token, row_slot,
                     token_slot_row);
  return hipGetLastError();
}

static int gather_grid(int64_t max_rows) {
  const int64_t blocks = (max_rows + 3) / 4;
  return static_cast<int>(blocks < 8192 ? (blocks > 0 ? blocks : 1) : 8192);
}

// Waves per row of the quantising gathers: enough for ~2048 waves in all, at
// most one per 64-lane pass of a row (H / 512 passes).
static int gather_parts(int64_t max_rows, int H) {
  const int64_t passes = (H / 8 + kWave - 1) / kWave;
  const int64_t want = (2048 + max_rows - 1) / (max_rows > 0 ? max_rows : 1);
  const int64_t p = want < passes ? want : passes;
  return static_cast<int>(p > 1 ? p : 1);
}

// Blocks of 4 waves for max_rows rows of `parts` waves each.
static int gather_grid_parts(int64_t max_rows, int parts) {
  const int64_t blocks = (max_rows * parts + 3) / 4;
  return static_cast<int>(blocks < 8192 ? (blocks > 0 ? blocks : 1) : 8192);
}

template <int KMAX>
static void launch_front_k(int qkind, dim3 grid, size_t lds, hipStream_t s,
                           const int32_t* topk_ids, int T, int k, int e_lo, int E_L, int cap,
                           int32_t* counts, int32_t* offsets, int32_t* row_token,
                           int32_t* row_slot, int32_t* token_slot_row, int tile_m, int4* info,
                           int32_t* n_tiles, int32_t* sync, int32_t* status, const uint4* x,
                           int H, int parts, uint2* xq, void* xq_scale) {
  auto kern = qkind == 1 ? index_front_kernel<KMAX, 1>
            : qkind == 2 ? index_front_kernel<KMAX, 2> : index_front_kernel<KMAX, 0>;
  hipLaunchKernelGGL(kern, grid, dim3(1024), lds, s, topk_ids, T, k, e_lo, E_L, cap, counts,
                     offsets, row_token, row_slot, token_slot_row, tile_m, info, n_tiles, sync,
                     status, x, H, parts, xq, xq_scale);
}

hipError_t launch_index_front(const int32_t* topk_ids, int T, int k, int e_lo, int E_L, int cap,
                              int32_t* counts, int32_t* offsets, int32_t* row_token,
                              int32_t* row_slot, int32_t* token_slot_row, int tile_m, int4* info,
                              int32_t* n_tiles, int32_t* sync, int32_t* status, int qkind,
                              const void* x, int H, void* xq, void* xq_scale, hipStream_t s) {
  if (T < 1 || T > kTokBlock || E_L < 1 || E_L > 1024 || tile_m < 1 || qkind < 0 || qkind > 2)
    return hipErrorInvalidValue;
  const size_t lds = static_cast<size_t>(E_L) * (kMaskWords + 1) * sizeof(uint32_t);
  const int parts = qkind ? gather_parts(T, H) : 1;
  const int qblocks = qkind ? ceil_div(T * parts, 16) : 0;
  const dim3 grid(static_cast<unsigned>(1 + qblocks));
  const uint4* xs = static_cast<const uint4*>(x);
  uint2* xd = static_cast<uint2*>(xq);
  if (k <= 8)
    launch_front_k<8>(qkind, grid, lds, s, topk_ids, T, k, e_lo, E_L, cap, counts, offsets,
                      row_token, row_slot, token_slot_row, tile_m, info, n_tiles, sync, status,
                      xs, H, parts, xd, xq_scale);
  else
    launch_front_k<32>(qkind, grid, lds, s, topk_ids, T, k, e_lo, E_L, cap, counts, offsets,
                       row_token, row_slot, token_slot_row, tile_m, info, n_tiles, sync, status,
                       xs, H, parts, xd, xq_scale);
  return hipGetLastError();
}

hipError_t launch_gather_bf16(const void* src, const int32_t* rows, const int32_t* n_rows,
                              int64_t max_rows, int H, void* dst, int64_t panel_rows,
                              hipStream_t s, const int32_t* counts, int cap) {
  if (panel_rows > 0)
    hipLaunchKernelGGL(gather_rows_panel_kernel,
                       dim3(gather_grid((max_rows + 15) / 16 * ((H / 32 + 7) / 8))),
                       dim3(256), 0, s, static_cast<const uint4*>(src), rows, n_rows,
                       static_cast<int>(max_rows), H / 8, panel_rows, counts, cap,
                       static_cast<uint4*>(dst));
  else
    hipLaunchKernelGGL(gather_rows_bf16_kernel, dim3(gather_grid(max_rows)), dim3(256), 0, s,
                       static_cast<const uint4*>(src), rows, n_rows, static_cast<int>(max_rows),
                       H / 8, counts, cap, static_cast<uint4*>(dst));
  return hipGetLastError();
}

hipError_t launch_pack_panel(const void* src, int64_t batch, int64_t rows, int64_t cols,
                             void* dst, hipStream_t s) {
  const int64_t units = batch * rows * (cols / 8);
  const int64_t blocks = (units + 255) / 256;
  hipLaunchKernelGGL(pack_panel_kernel, dim3(static_cast<unsigned>(blocks < 16384 ? blocks : 16384)),
                     dim3(256), 0, s, static_cast<const uint4*>(src), batch, rows, cols,
                     static_cast<uint4*>(dst));
  return hipGetLastError();
}

hipError_t launch_pack_scales_mx(const void* src, int64_t batch, int64_t rows, int64_t cols,
                                 void* dst, hipStream_t s) {
  const int64_t units = batch * rows * (cols / 128);
  const int64_t blocks = (units + 255) / 256;
  hipLaunchKernelGGL(pack_scales_mx_kernel,
                     dim3(static_cast<unsigned>(blocks < 16384 ? blocks : 16384)), dim3(256), 0, s,
                     static_cast<const uint32_t*>(src), batch, rows, cols / 128,
                     static_cast<uint32_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_gather_fp8(const void* src, const int32_t* rows, const int32_t* n_rows,
                             int64_t max_rows, int H, void* dst, float* dst_scale,
                             hipStream_t s, const int32_t* counts, int cap) {
  const int parts = gather_parts(max_rows, H);
  hipLaunchKernelGGL(gather_rows_fp8_kernel, dim3(gather_grid_parts(max_rows, parts)), dim3(256),
                     0, s, static_cast<const uint4*>(src), rows, n_rows,
                     static_cast<int>(max_rows), H, parts, counts, cap,
                     static_cast<uint2*>(dst), dst_scale);
  return hipGetLastError();
}

hipError_t launch_quant_blocks(const void* src, int64_t batch, int64_t rows, int64_t cols,
                               void* codes, float* scales, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(cols / 128), static_cast<unsigned>((rows + 127) / 128),
                  static_cast<unsigned>(batch));
  hipLaunchKernelGGL(quant_blocks_kernel, grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(src), rows, cols,
                     static_cast<uint8_t*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_quant_mx4(const void* src, int64_t rows, int64_t cols, void* codes,
                            uint8_t* scales, hipStream_t s) {
  const int64_t blocks = rows * (cols / 32);
  const int64_t grid = (blocks + 255) / 256;
  hipLaunchKernelGGL(quant_mx4_kernel, dim3(static_cast<unsigned>(grid < 65536 ? grid : 65536)),
                     dim3(256), 0, s, static_cast<const uint4*>(src), blocks,
                     static_cast<uint4*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_gather_mx8(const void* src, const int32_t* rows, const int32_t* n_rows,
                             int64_t max_rows, int H, void* dst, uint8_t* dst_scale,
                             hipStream_t s, const int32_t* counts, int cap) {
  const int parts = gather_parts(max_rows, H);
  hipLaunchKernelGGL(gather_rows_mx8_kernel, dim3(gather_grid_parts(max_rows, parts)), dim3(256),
                     0, s, static_cast<const uint4*>(src), rows, n_rows,
                     static_cast<int>(max_rows), H, parts, counts, cap,
                     static_cast<uint2*>(dst), dst_scale);
  return hipGetLastError();
}

}  // namespace moe
