// Grouped expert GEMMs of the MoE FFN on the gfx950 matrix cores (MFMA).
//
// Page "OverlapAdvisor: Modeling and Adapting Computation-Communication
// Overlap for Distributed MoE Serving": section 4.2.2 / Eq. 8 (the up
// GroupGEMM of a gated MLP has m = 2 first-layer matrices, 2 m H I FLOPs per
// row; the down GroupGEMM 2 H I), Table 6 (gated SwiGLU); section 5.1 (tile
// counts W1, W2 per expert from B_M x B_N tiles).  Page "CascadeEP ...",
// Appendix C (groups aligned to the GEMM tile; the two expert GEMMs with the
// activation and quantisation between them).  Page "ExpertPlex", Eq. 3
// (tile-aware token count: sum over experts of ceil(m_e / M_t)).
//
// Tile schedule.  One block turns the device-resident expert offsets into a
// table of 128-row m-tiles -- ceil(n_e / 128) per expert, none for an empty
// expert -- and their count.  The GEMM grid is an upper bound; each block
// derives its tile from the live count, so data-dependent sizes never go
// back to the host.  Tiles are ordered expert by expert, n-tile by n-tile,
// m-tile fastest, so consecutive tiles share one weight tile (and an
// expert's activation rows); that order is cut into 8 contiguous ranges, one
// per XCD (blocks are dispatched to the 8 XCDs round-robin by id), so the
// blocks sharing a weight tile run on the same XCD and meet in its L2.
//
// Block tile: 128 token rows x 256 weight rows, 4 waves as 2 (rows) x 2
// (weights), each wave 64 x 128 = 2 x 4 MFMA 32x32 tiles.  The weight tile is
// the MFMA A operand and the token tile the B operand, so a lane's
// accumulator holds 4 consecutive output columns of one token row.  Both
// tiles go global -> registers -> LDS, double buffered: the loads of step
// k+1 are in flight while step k runs on the matrix cores.  The LDS row pitch
// is padded by 16 bytes, which puts the 16-byte fragment reads of 16
// consecutive rows on disjoint banks.
//
// SwiGLU mode: the 256 weight rows are 128 gate rows and the 128 matching up
// rows, arranged so each wave holds the gate and up accumulators of the same
// (row, column) in the same lane; the epilogue forms h = silu(gate) * up and
// never writes the [n, 2I] product.  With block-FP8 output the block's 128 h
// columns are exactly one quantisation group: the two waves sharing a row
// range exchange their row maxima through LDS and the epilogue writes E4M3
// codes and the per-row group scale straight from the fp32 values.
//
// Block-FP8 operands: one K step is one 128-wide scale block; its products go
// to a zeroed temporary that is added to the accumulator times
// (weight block scale x token group scale).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kBM = 128;      // token rows per block
constexpr int kBN = 256;      // weight rows per block
constexpr int kThreads = 256;
constexpr int kXcds = 8;

enum { MODE_PLAIN = 0, MODE_SWIGLU = 1, MODE_SWIGLU_FP8OUT = 2 };

struct GemmArgs {
  const uint8_t* A;        // activations [N_cap, K] (bf16 or e4m3)
  const float* A_scale;    // fp8: [N_cap, K/128]
  const uint8_t* W;        // weights [E_L][NW][K]
  const float* W_scale;    // fp8: [E_L][NW/128][K/128]
  void* C;                 // [N_cap, Nout] bf16, or e4m3 in MODE_SWIGLU_FP8OUT
  float* C_scale;          // MODE_SWIGLU_FP8OUT: [N_cap, Nout/128]
  const int32_t* offsets;  // [E_L + 1]
  const int4* info;        // per m-tile {expert, first m-tile of expert, m-tiles of expert, 0}
  const int32_t* n_tiles;  // live m-tiles
  int K, Nout, NW, nt_n;   // NW = 2 Nout (SwiGLU) or Nout; nt_n n-tiles per expert
  int64_t w_stride;        // bytes per expert of W
  int64_t ws_stride;       // floats per expert of W_scale
};

__global__ __launch_bounds__(1024) void tile_schedule_kernel(
    const int32_t* __restrict__ offsets, int E_L, int4* __restrict__ info,
    int32_t* __restrict__ n_tiles) {
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E_L) cnt = offsets[e + 1] - offsets[e];
  const int tiles = ceil_div(cnt, kBM);
  int total;
  const int start = block_exclusive_scan(tiles, &total);
  if (e < E_L)
    for (int i = 0; i < tiles; ++i) info[start + i] = make_int4(e, start, tiles, 0);
  if (e == 0) *n_tiles = total;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

template <int ROWB>
struct Stage {
  static constexpr int kPitch = ROWB + 16;
  static constexpr int kBytes = (kBM + kBN) * kPitch;
  static constexpr int kChunks = ROWB / 16;            // 16-byte chunks per row
  static constexpr int kLdA = kBM * kChunks / kThreads;
  static constexpr int kLdW = kBN * kChunks / kThreads;
};

// Global -> register -> LDS staging of one K step of both tiles.
template <int ROWB>
struct Loader {
  using S = Stage<ROWB>;
  const uint8_t* gA[S::kLdA];
  const uint8_t* gW[S::kLdW];
  int oA[S::kLdA], oW[S::kLdW];
  uint4 rA[S::kLdA], rW[S::kLdW];

  __device__ __forceinline__ void init(const GemmArgs& g, int swiglu, const uint8_t* We,
                                       int64_t ldb, int nt, int row0, int row_end) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < S::kLdA; ++i) {
      const int c = tid + kThreads * i;
      const int r = c / S::kChunks, col = (c % S::kChunks) * 16;
      gA[i] = g.A + static_cast<int64_t>(min(row0 + r, row_end - 1)) * ldb + col;
      oA[i] = r * S::kPitch + col;
    }
#pragma unroll
    for (int i = 0; i < S::kLdW; ++i) {
      const int c = tid + kThreads * i;
      const int r = c / S::kChunks, col = (c % S::kChunks) * 16;
      int wrow;
      if (swiglu)
        wrow = r < kBN / 2 ? nt * (kBN / 2) + r : g.Nout + nt * (kBN / 2) + (r - kBN / 2);
      else
        wrow = min(nt * kBN + r, g.NW - 1);
      gW[i] = We + static_cast<int64_t>(wrow) * ldb + col;
      oW[i] = (kBM + r) * S::kPitch + col;
    }
  }
  __device__ __forceinline__ void load(int64_t kbyte) {
#pragma unroll
    for (int i = 0; i < S::kLdW; ++i) rW[i] = *reinterpret_cast<const uint4*>(gW[i] + kbyte);
#pragma unroll
    for (int i = 0; i < S::kLdA; ++i) rA[i] = *reinterpret_cast<const uint4*>(gA[i] + kbyte);
  }
  __device__ __forceinline__ void store(uint8_t* s) {
#pragma unroll
    for (int i = 0; i < S::kLdW; ++i) *reinterpret_cast<uint4*>(s + oW[i]) = rW[i];
#pragma unroll
    for (int i = 0; i < S::kLdA; ++i) *reinterpret_cast<uint4*>(s + oA[i]) = rA[i];
  }
};

// LDS row (within the weight tile) of the wave's weight block i (0..3).
__device__ __forceinline__ int wblock_row(int swiglu, int wn, int i) {
  if (swiglu) return (i < 2 ? 0 : kBN / 2) + wn * 64 + (i & 1) * 32;
  return wn * 128 + i * 32;
}

template <bool FP8, int MODE, int ROWB>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(const GemmArgs g) {
  using S = Stage<ROWB>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float row_amax[2][kBM];
  constexpr bool kSwiglu = MODE != MODE_PLAIN;

  // ---- which tile ----
  const int total = *g.n_tiles * g.nt_n;
  const int per_xcd = ceil_div(total, kXcds);
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int t = (blockIdx.x % kXcds) * per_xcd + slot;
  if (t >= total) return;
  const int4 inf = g.info[t / g.nt_n];
  const int e = inf.x, u = t - inf.y * g.nt_n;
  const int nt = u / inf.z, mt = u % inf.z;
  const int seg_end = g.offsets[e + 1];
  const int row0 = g.offsets[e] + mt * kBM;

  const int64_t ldb = FP8 ? g.K : 2ll * g.K;  // bytes per row of A and W
  const uint8_t* We = g.W + e * g.w_stride;
  Loader<ROWB> ld;
  ld.init(g, kSwiglu, We, ldb, nt, row0, seg_end);

  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int lr = lane & 31;
  const int kq = (lane >> 5) * (FP8 ? 32 : 16);  // byte offset of the lane's k values
  int offW[4], offA[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) offW[i] = (kBM + wblock_row(kSwiglu, wn, i) + lr) * S::kPitch + kq;
#pragma unroll
  for (int j = 0; j < 2; ++j) offA[j] = (wm * 64 + j * 32 + lr) * S::kPitch + kq;

  // fp8 scale rows
  const float* swp[4];
  const float* sxp[2];
  if (FP8) {
    const int kb_n = g.K / 128;
    const float* wsc = g.W_scale + e * g.ws_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lrow = wblock_row(kSwiglu, wn, i);
      int grow;
      if (kSwiglu)
        grow = lrow < kBN / 2 ? nt * (kBN / 2) + lrow : g.Nout + nt * (kBN / 2) + (lrow - kBN / 2);
      else
        grow = min(nt * kBN + lrow, g.NW - 1);
      swp[i] = wsc + static_cast<int64_t>(grow / 128) * kb_n;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
      sxp[j] = g.A_scale + static_cast<int64_t>(min(row0 + wm * 64 + j * 32 + lr, seg_end - 1)) * kb_n;
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = static_cast<int>(ldb / ROWB);
  ld.load(0);
  ld.store(smem);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const uint8_t* s = smem + (kt & 1) * S::kBytes;
    if (kt + 1 < nk) ld.load(static_cast<int64_t>(kt + 1) * ROWB);
    if constexpr (!FP8) {
#pragma unroll
      for (int kk = 0; kk < ROWB / 32; ++kk) {  // 16 bf16 (32 bytes) per MFMA
        bf16x8 a[4], b[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8*>(s + offW[i] + kk * 32);
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const bf16x8*>(s + offA[j] + kk * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    } else {
      float sw[4], sx[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) sw[i] = swp[i][kt];
#pragma unroll
      for (int j = 0; j < 2; ++j) sx[j] = sxp[j][kt];
      f32x16 tmp[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) tmp[i][j][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {  // 64 e4m3 (64 bytes) per MFMA
        i32x8 a[4], b[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const i32x4 lo = *reinterpret_cast<const i32x4*>(s + offW[i] + kk * 64);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(s + offW[i] + kk * 64 + 16);
          a[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const i32x4 lo = *reinterpret_cast<const i32x4*>(s + offA[j] + kk * 64);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(s + offA[j] + kk * 64 + 16);
          b[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            tmp[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], tmp[i][j], 0,
                                                                        0, 0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float sc = sw[i] * sx[j];
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] += tmp[i][j][r] * sc;
        }
    }
    if (kt + 1 < nk) ld.store(smem + ((kt + 1) & 1) * S::kBytes);
    __syncthreads();
  }

  // ---- epilogue ----
  // Accumulator element q*4 + r of a 32x32 tile is weight row q*8 + (lane/32)*4
  // + r and token row lane % 32.
  const int cq = (lane >> 5) * 4;
  if constexpr (MODE == MODE_PLAIN) {
    uint16_t* C = static_cast<uint16_t*>(g.C);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = row0 + wm * 64 + j * 32 + lr;
      if (m >= seg_end) continue;
      uint16_t* crow = C + static_cast<int64_t>(m) * g.Nout;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nt * kBN + wn * 128 + i * 32 + q * 8 + cq;
          if (col >= g.Nout) continue;
          uint2 o;
          o.x = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
          o.y = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
          *reinterpret_cast<uint2*>(crow + col) = o;
        }
    }
  } else {
    // h = silu(gate) * up, kept in acc[hb][j] (hb = 0, 1).
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[hb][j][r] = silu_mul(acc[hb][j][r], acc[hb + 2][j][r]);
    if constexpr (MODE == MODE_SWIGLU) {
      uint16_t* C = static_cast<uint16_t*>(g.C);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = row0 + wm * 64 + j * 32 + lr;
        if (m >= seg_end) continue;
        uint16_t* crow = C + static_cast<int64_t>(m) * g.Nout;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint2 o;
            o.x = pack_bf16x2(acc[hb][j][q * 4 + 0], acc[hb][j][q * 4 + 1]);
            o.y = pack_bf16x2(acc[hb][j][q * 4 + 2], acc[hb][j][q * 4 + 3]);
            *reinterpret_cast<uint2*>(crow + nt * 128 + wn * 64 + hb * 32 + q * 8 + cq) = o;
          }
      }
    } else {
      // One 128-column group per row: this wave holds 64 of its columns.
      float amax[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float m = 0.0f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[hb][j][r]));
        m = fmaxf(m, __shfl_xor(m, 32));
        amax[j] = m;
        if (lane < 32) row_amax[wn][wm * 64 + j * 32 + lr] = m;
      }
      __syncthreads();
      uint8_t* C = static_cast<uint8_t*>(g.C);
      const int groups = g.Nout / 128;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int lrow = wm * 64 + j * 32 + lr;
        const float am = fmaxf(amax[j], row_amax[wn ^ 1][lrow]);
        const float sc = am > 0.0f ? am / 448.0f : 1.0f;
        const int m = row0 + lrow;
        if (m >= seg_end) continue;
        uint8_t* crow = C + static_cast<int64_t>(m) * g.Nout;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t v = f32x4_to_e4m3x4(acc[hb][j][q * 4 + 0] / sc, acc[hb][j][q * 4 + 1] / sc,
                                               acc[hb][j][q * 4 + 2] / sc, acc[hb][j][q * 4 + 3] / sc);
            *reinterpret_cast<uint32_t*>(crow + nt * 128 + wn * 64 + hb * 32 + q * 8 + cq) = v;
          }
        if (wn == 0 && lane < 32) g.C_scale[static_cast<int64_t>(m) * groups + nt] = sc;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined kernel (bf16 and block-FP8).  Same tile and operand layout as
// grouped_gemm_kernel; the K loop runs a three-stage LDS ring fed by
// direct-to-LDS buffer loads (global memory -> LDS without registers):
//   * the loads of K step kt+3 are issued right after the barrier that ends
//     step kt, so two steps of loads are always in flight behind the one
//     being computed; each wave counts its own loads (s_waitcnt vmcnt) and
//     one barrier per step publishes a stage to all four waves;
//   * a direct load writes 1 KB of LDS per wave instruction (16 bytes per
//     lane), i.e. 8 tile rows of 128 bytes; the lane -> global chunk map
//     applies the swizzle chunk ^ ((row >> 1) & 7), which makes the 16-byte
//     fragment reads of 16 consecutive rows hit disjoint LDS banks;
//   * operand fragments are double-buffered in registers (the LDS reads of
//     sub-step kk+1 are issued between the MFMAs of sub-step kk), and the
//     last sub-step's MFMAs straddle the step barrier so that they cover the
//     first fragment reads of the next stage;
//   * buffer loads take a scalar base and 32-bit lane offsets; rows past the
//     expert's segment lie outside the buffer's range and read as zero.
// ---------------------------------------------------------------------------
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kStages = 3;
constexpr int kRowBytes = 128;                           // K bytes per row per step
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;     // 48 KB
constexpr int kWRegion = kBM * kRowBytes;                // weight rows start here
constexpr int kDmaPerWave = (kBM + kBN) / 8 / 4;         // 12 loads of 8 rows per wave

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                           kBufFlags);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding),
// and the same with every LDS access of the wave also complete.
#define WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | 0x70 | 0xF00 | ((((n) >> 4) & 3) << 14))
#define WAIT_VMCNT_LDS(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | 0x70 | ((((n) >> 4) & 3) << 14))
#define SCHED(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <bool FP8, int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_pipelined_kernel(const GemmArgs g) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  __shared__ float row_amax[2][kBM];
  constexpr bool kSwiglu = MODE != MODE_PLAIN;
  constexpr int kKK = FP8 ? 2 : 4;             // MFMA sub-steps per K step
  constexpr int kScaleLoads = FP8 ? 6 : 0;     // per-step scale loads per lane
  constexpr int kWaitStep = kDmaPerWave + kScaleLoads;

  const int total = *g.n_tiles * g.nt_n;
  const int per_xcd = ceil_div(total, kXcds);
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int t = (blockIdx.x % kXcds) * per_xcd + slot;
  if (t >= total) return;
  const int4 inf = g.info[t / g.nt_n];
  const int e = inf.x, u = t - inf.y * g.nt_n;
  const int nt = u / inf.z, mt = u % inf.z;
  const int seg_end = g.offsets[e + 1];
  const int row0 = g.offsets[e] + mt * kBM;

  const int ldb = FP8 ? g.K : 2 * g.K;  // bytes per row of A and W
  const int nk = ldb / kRowBytes;
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc(g.A + static_cast<int64_t>(row0) * ldb, static_cast<int64_t>(seg_end - row0) * ldb);
  const __amdgpu_buffer_rsrc_t rW =
      make_rsrc(g.W + e * g.w_stride, static_cast<int64_t>(g.NW) * ldb);

  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  // ---- direct-load assignment: wave w moves 8-row groups w*4+q (A) and
  // 16 + w*8 + q (W) of the 48 groups of a stage.
  int voff[kDmaPerWave];
  int ldst[kDmaPerWave];  // byte offset of the group within a stage
#pragma unroll
  for (int q = 0; q < kDmaPerWave; ++q) {
    const int grp = q < 4 ? w * 4 + q : 16 + w * 8 + (q - 4);
    const int rr = grp * 8 + (lane >> 3);           // row within the stage (A rows, then W rows)
    const int chunk = (lane & 7) ^ ((rr >> 1) & 7);
    int grow;
    if (rr < kBM) {
      grow = rr;
    } else {
      const int r = rr - kBM;
      if (kSwiglu)
        grow = r < kBN / 2 ? nt * (kBN / 2) + r : g.Nout + nt * (kBN / 2) + (r - kBN / 2);
      else
        grow = min(nt * kBN + r, g.NW - 1);
    }
    voff[q] = grow * ldb + chunk * 16;
    ldst[q] = grp * 1024;
  }
  auto dma = [&](int step, int stage) {
    const int soff = min(step, nk - 1) * kRowBytes;
    uint8_t* base = smem + stage * kStageBytes;
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(q < 4 ? rA : rW, (lds_ptr_t)(base + ldst[q]), 16,
                                               voff[q], soff, 0, 0);
  };

  // ---- fragment addressing
  const int wm = w & 1, wn = w >> 1;
  const int lr = lane & 31, hi = lane >> 5, sl = (lr >> 1) & 7;
  int foff[4];  // per-lane byte offset inside a 32-row block for the sub-step's chunk(s)
  if (!FP8) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) foff[kk] = lr * kRowBytes + (((2 * kk) | hi) ^ sl) * 16;
  } else {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c0 = (4 * kk + 2 * hi) ^ sl;
      foff[2 * kk] = lr * kRowBytes + c0 * 16;
      foff[2 * kk + 1] = lr * kRowBytes + (c0 ^ 1) * 16;
    }
  }
  int wbase[4], abase[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) wbase[i] = kWRegion + wblock_row(kSwiglu, wn, i) * kRowBytes;
#pragma unroll
  for (int j = 0; j < 2; ++j) abase[j] = (wm * 64 + j * 32) * kRowBytes;

  // ---- fp8 scales
  const float* swp[4];
  const float* sxp[2];
  float sw[4], sx[2];
  if (FP8) {
    const int kb_n = g.K / 128;
    const float* wsc = g.W_scale + e * g.ws_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lrow = wblock_row(kSwiglu, wn, i);
      int grow;
      if (kSwiglu)
        grow = lrow < kBN / 2 ? nt * (kBN / 2) + lrow : g.Nout + nt * (kBN / 2) + (lrow - kBN / 2);
      else
        grow = min(nt * kBN + lrow, g.NW - 1);
      swp[i] = wsc + static_cast<int64_t>(grow / 128) * kb_n;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
      sxp[j] = g.A_scale +
               static_cast<int64_t>(min(row0 + wm * 64 + j * 32 + lr, seg_end - 1)) * kb_n;
  }
  auto load_scales = [&](int step) {
    if (FP8) {
      const int k = min(step, nk - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) sw[i] = swp[i][k];
#pragma unroll
      for (int j = 0; j < 2; ++j) sx[j] = sxp[j][k];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // fragments: bf16 uses 4 dwords per operand, fp8 8 dwords
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type frag_t;
  frag_t fa[2][4], fb[2][2];
  auto rd16 = [&](const uint8_t* p) { return *reinterpret_cast<const i32x4*>(p); };
  auto lfrag = [&](const uint8_t* st, int kk, int set) {
    if constexpr (!FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[set][i] = *reinterpret_cast<const bf16x8*>(st + wbase[i] + foff[kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[set][j] = *reinterpret_cast<const bf16x8*>(st + abase[j] + foff[kk]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x4 lo = rd16(st + wbase[i] + foff[2 * kk]), hi4 = rd16(st + wbase[i] + foff[2 * kk + 1]);
        fa[set][i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const i32x4 lo = rd16(st + abase[j] + foff[2 * kk]), hi4 = rd16(st + abase[j] + foff[2 * kk + 1]);
        fb[set][j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      }
    }
  };
  f32x16 tmp[4][2];
  auto zero_tmp = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmp[i][j][r] = 0.0f;
  };
  auto mma = [&](int set, int first, int count) {
#pragma unroll
    for (int q = first; q < first + count; ++q) {
      const int i = q >> 1, j = q & 1;
      if constexpr (!FP8)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
      else
        tmp[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[set][i], fb[set][j],
                                                                    tmp[i][j], 0, 0, 0, 0, 0, 0);
    }
  };
  auto scale_acc = [&]() {
    if constexpr (FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float sc = sw[i] * sx[j];
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] += tmp[i][j][r] * sc;
        }
    }
  };

  // ---- prologue: steps 0, 1 (+ scales of step 0), 2 in flight
  dma(0, 0);
  dma(1, 1);
  load_scales(0);
  dma(2, 2);
  WAIT_VMCNT(kDmaPerWave + kScaleLoads + kDmaPerWave);
  __builtin_amdgcn_s_barrier();
  lfrag(smem, 0, 0);

  for (int kt = 0; kt < nk; ++kt) {
    const int cur_stage = kt % kStages;
    const uint8_t* cur = smem + cur_stage * kStageBytes;
    const uint8_t* nxt = smem + ((kt + 1) % kStages) * kStageBytes;
    if (FP8) zero_tmp();
#pragma unroll
    for (int kk = 0; kk + 1 < kKK; ++kk) {
      lfrag(cur, kk + 1, (kk + 1) & 1);
      mma(kk & 1, 0, 8);
#pragma unroll
      for (int q = 0; q < (FP8 ? 8 : 6); ++q) {
        SCHED(kSchedMfma, 1);
        SCHED(kSchedDsRead, 1);
      }
      if (!FP8) SCHED(kSchedMfma, 2);
    }
    constexpr int last = (kKK - 1) & 1;
    mma(last, 0, 4);
    // Step boundary: this wave's loads of step kt+1 have landed once at most
    // the later group (scales of kt+1 if fp8, loads of kt+2) is in flight,
    // and its own reads of stage kt are done before anyone refills it.
    WAIT_VMCNT_LDS(kWaitStep);
    __builtin_amdgcn_s_barrier();
    // Stage kt is free in every wave now; refill it with step kt+3.
    lfrag(nxt, 0, 0);
    mma(last, 4, 4);
    if (FP8) {
      scale_acc();
      load_scales(kt + 1);
    }
    dma(kt + 3, cur_stage);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      SCHED(kSchedDsRead, FP8 ? 3 : 2);
      SCHED(kSchedMfma, 1);
      SCHED(kSchedVmemRead, 3);
    }
  }
  WAIT_VMCNT(0);

  // ---- epilogue (accumulator element q*4 + r of a 32x32 tile is weight row
  // q*8 + (lane/32)*4 + r and token row lane % 32)
  const int cq = (lane >> 5) * 4;
  if constexpr (MODE == MODE_PLAIN) {
    uint16_t* C = static_cast<uint16_t*>(g.C);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = row0 + wm * 64 + j * 32 + lr;
      if (m >= seg_end) continue;
      uint16_t* crow = C + static_cast<int64_t>(m) * g.Nout;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nt * kBN + wn * 128 + i * 32 + q * 8 + cq;
          if (col >= g.Nout) continue;
          uint2 o;
          o.x = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
          o.y = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
          *reinterpret_cast<uint2*>(crow + col) = o;
        }
    }
  } else {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[hb][j][r] = silu_mul(acc[hb][j][r], acc[hb + 2][j][r]);
    if constexpr (MODE == MODE_SWIGLU) {
      uint16_t* C = static_cast<uint16_t*>(g.C);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = row0 + wm * 64 + j * 32 + lr;
        if (m >= seg_end) continue;
        uint16_t* crow = C + static_cast<int64_t>(m) * g.Nout;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint2 o;
            o.x = pack_bf16x2(acc[hb][j][q * 4 + 0], acc[hb][j][q * 4 + 1]);
            o.y = pack_bf16x2(acc[hb][j][q * 4 + 2], acc[hb][j][q * 4 + 3]);
            *reinterpret_cast<uint2*>(crow + nt * 128 + wn * 64 + hb * 32 + q * 8 + cq) = o;
          }
      }
    } else {
      float amax[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float m = 0.0f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[hb][j][r]));
        m = fmaxf(m, __shfl_xor(m, 32));
        amax[j] = m;
        if (lane < 32) row_amax[wn][wm * 64 + j * 32 + lr] = m;
      }
      __syncthreads();
      uint8_t* C = static_cast<uint8_t*>(g.C);
      const int groups = g.Nout / 128;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int lrow = wm * 64 + j * 32 + lr;
        const float am = fmaxf(amax[j], row_amax[wn ^ 1][lrow]);
        const float sc = am > 0.0f ? am / 448.0f : 1.0f;
        const int m = row0 + lrow;
        if (m >= seg_end) continue;
        uint8_t* crow = C + static_cast<int64_t>(m) * g.Nout;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t v = f32x4_to_e4m3x4(acc[hb][j][q * 4 + 0] / sc, acc[hb][j][q * 4 + 1] / sc,
                                               acc[hb][j][q * 4 + 2] / sc, acc[hb][j][q * 4 + 3] / sc);
            *reinterpret_cast<uint32_t*>(crow + nt * 128 + wn * 64 + hb * 32 + q * 8 + cq) = v;
          }
        if (wn == 0 && lane < 32) g.C_scale[static_cast<int64_t>(m) * groups + nt] = sc;
      }
    }
  }
}

template <bool FP8, int MODE>
hipError_t launch_pipelined(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  auto kern = gemm_pipelined_kernel<FP8, MODE>;
  const size_t lds = kStages * kStageBytes;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
      (void)hipGetLastError();
    attr_set = true;
  }
  const int64_t blocks = (max_tiles * g.nt_n + kXcds - 1) / kXcds * kXcds + kXcds;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), lds, s, g);
  return hipGetLastError();
}

template <bool FP8, int MODE, int ROWB>
hipError_t launch_one(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  auto kern = grouped_gemm_kernel<FP8, MODE, ROWB>;
  const size_t lds = 2 * Stage<ROWB>::kBytes;
  // Allow more than 64 KB of dynamic LDS (gfx950 has 160 KB per CU).  If
  // the runtime refuses, the launch below reports the problem.
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
      (void)hipGetLastError();
    attr_set = true;
  }
  // Enough blocks for every live tile after the per-XCD split.
  const int64_t blocks = (max_tiles * g.nt_n + kXcds - 1) / kXcds * kXcds + kXcds;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), lds, s, g);
  return hipGetLastError();
}

}  // namespace

int64_t max_m_tiles(int64_t n_cap, int E_L) { return ceil_div<int64_t>(n_cap, kBM) + E_L; }

hipError_t launch_tile_schedule(const int32_t* offsets, int E_L, int4* info, int32_t* n_tiles,
                                hipStream_t s) {
  hipLaunchKernelGGL(tile_schedule_kernel, dim3(1), dim3(1024), 0, s, offsets, E_L, info, n_tiles);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmLaunch& L, hipStream_t s) {
  GemmArgs g{};
  g.A = static_cast<const uint8_t*>(L.A);
  g.A_scale = L.A_scale;
  g.W = static_cast<const uint8_t*>(L.W);
  g.W_scale = L.W_scale;
  g.C = L.C;
  g.C_scale = L.C_scale;
  g.offsets = L.offsets;
  g.info = L.info;
  g.n_tiles = L.n_tiles;
  g.K = L.K;
  g.Nout = L.Nout;
  g.NW = L.swiglu ? 2 * L.Nout : L.Nout;
  g.nt_n = L.swiglu ? L.Nout / (kBN / 2) : ceil_div(L.Nout, kBN);
  const int64_t elem = L.fp8 ? 1 : 2;
  g.w_stride = static_cast<int64_t>(g.NW) * L.K * elem;
  g.ws_stride = L.fp8 ? static_cast<int64_t>(g.NW / 128) * (L.K / 128) : 0;
  if (!L.fp8) {
    if (L.swiglu) return launch_pipelined<false, MODE_SWIGLU>(g, L.max_tiles, s);
    return launch_pipelined<false, MODE_PLAIN>(g, L.max_tiles, s);
  }
  if (L.swiglu) {
    if (L.C_scale) return launch_pipelined<true, MODE_SWIGLU_FP8OUT>(g, L.max_tiles, s);
    return launch_pipelined<true, MODE_SWIGLU>(g, L.max_tiles, s);
  }
  return launch_pipelined<true, MODE_PLAIN>(g, L.max_tiles, s);
}

}  // namespace moe
