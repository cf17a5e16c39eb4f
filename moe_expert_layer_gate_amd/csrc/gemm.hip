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
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kBM = 128;      // token rows per block
constexpr int kBN = 256;      // weight rows per block
constexpr int kThreads = 256;
constexpr int kXcds = 8;

enum { MODE_PLAIN = 0, MODE_SWIGLU = 1, MODE_SWIGLU_FP8OUT = 2, MODE_GELU = 3,
       MODE_SWIGLU_MX8OUT = 4 };

// GELU, a * Phi(a) = a erfc(-a / sqrt 2) / 2, in fp32 (the up GEMM's epilogue
// of the standard MLP).  erfc from the rational-exponential approximation of
// Abramowitz and Stegun, Handbook of Mathematical Functions, 7.1.26 (erf to
// within 1.5e-7 absolute): erfc(x) = t (a1 + t (a2 + t (a3 + t (a4 + t a5))))
// exp(-x^2), t = 1 / (1 + p x), for x >= 0, and 2 - erfc(-x) below -- one
// reciprocal and one exponential, a fifth of the cost of the library erfcf
// here (the h it feeds is rounded to bf16, 2^-9 relative).
__device__ __forceinline__ float gelu_f(float a) {
  const float x = -a * 0.70710678118654752f;
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);  // 1 ulp: ample here
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f +
                                                                         t * 1.061405429f))));
  const float q = poly * __expf(-ax * ax);  // erfc(|x|)
  return 0.5f * a * (x >= 0.0f ? q : 2.0f - q);
}
// The epilogue value of the plain-geometry modes: y as is, or gelu(h).
template <int MODE>
__device__ __forceinline__ float plain_act(float v) {
  if constexpr (MODE == MODE_GELU) return gelu_f(v);
  return v;
}

struct GemmArgs {
  const uint8_t* A;        // activations [N_cap, K] (bf16 or e4m3)
  const float* A_scale;    // fp8: [N_cap, K/128]
  const uint8_t* W;        // weights [E_L][NW][K]
  const float* W_scale;    // fp8: [E_L][NW/128][K/128]
  void* C;                 // [N_cap, Nout] bf16, or e4m3 in MODE_SWIGLU_FP8OUT
  float* C_scale;          // MODE_SWIGLU_FP8OUT: [N_cap, Nout/128]
  const int32_t* seg;      // segment table: offsets [E_L + 1], or counts [E_L]
  int seg_cap;             // 0: contiguous (offsets); > 0: masked blocks of seg_cap rows
  const int4* info;        // per m-tile {expert, first m-tile of expert, m-tiles of expert, 0}
  const int32_t* n_tiles;  // live m-tiles
  int K, Nout, NW, nt_n;   // NW = 2 Nout (SwiGLU) or Nout; nt_n n-tiles per expert
  int64_t w_stride;        // bytes per expert of W
  int64_t ws_stride;       // floats (MX: bytes) per expert of W_scale
  // Operand addressing: byte (row, c) of A or W is at row * rs + (c / 64) * cs
  // + c % 64 -- row major: rs = row bytes, cs = 64; panel layout: rs = 64,
  // cs = 64 * rows of the matrix.
  int a_rs, w_rs;
  int a_cs, w_cs;          // (a buffer's whole span stays below 2 GiB, see the host)
  // MX weight scales: byte (row, 4-byte piece p) at row * ws_rs + p * ws_cs --
  // row major: ws_rs = K / 32, ws_cs = 4; panel: ws_rs = 4, ws_cs = 4 NW.
  int ws_rs, ws_cs;
  int64_t a_bytes;         // size of the A buffer
  int64_t c_cs;            // SwiGLU bf16 output: 0 = row major, else panel stride
  const int32_t* a_index;  // fused gather: GEMM row j reads A row a_index[j]
  int32_t* tickets;        // persistent large-tile GEMM: one unit counter per XCD (zeroed
                           // by the schedule kernel), else null
};

// Byte offset of element (m, col) of a bf16 output with Nout columns.
__device__ __forceinline__ int64_t out_offset(const GemmArgs& g, int m, int col) {
  if (g.c_cs) return (col >> 5) * g.c_cs + static_cast<int64_t>(m) * 64 + (col & 31) * 2;
  return (static_cast<int64_t>(m) * g.Nout + col) * 2;
}

// Rows [x, y) of local expert e.  Contiguous layout (cap == 0): seg holds
// the offsets; masked layout: seg holds the counts and the expert's block
// starts at e * cap.
__device__ __forceinline__ int2 segment(const int32_t* seg, int cap, int e) {
  if (cap) return make_int2(e * cap, e * cap + seg[e]);
  return make_int2(seg[e], seg[e + 1]);
}

// The m-tile table of the paths without unit tables, from the segments
// (build_tile_table).
__global__ __launch_bounds__(1024) void tile_schedule_kernel(
    const int32_t* __restrict__ seg, int seg_cap, int E_L, int tile_m, int4* __restrict__ info,
    int32_t* __restrict__ n_tiles, int32_t* __restrict__ sync, int32_t* __restrict__ status) {
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E_L) {
    const int2 sg = segment(seg, seg_cap, e);
    cnt = sg.y - sg.x;
  }
  build_tile_table(e, E_L, cnt, tile_m, info, n_tiles, sync, status);
}

// silu(g) u = g u / (1 + exp(-g)) with the hardware reciprocal (1 ulp)
// instead of an IEEE division: h is rounded to bf16 or an 8-bit code at once.
// Large negative g: exp(-g) = inf, the reciprocal 0 and h -0, as the division
// gives.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// LDS row (within the weight tile) of the wave's weight block i (0..3).
__device__ __forceinline__ int wblock_row(int swiglu, int wn, int i) {
  if (swiglu) return (i < 2 ? 0 : kBN / 2) + wn * 64 + (i & 1) * 32;
  return wn * 128 + i * 32;
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
//   * buffer loads take a scalar base, moved on by one K step per step, and
//     32-bit lane offsets; the lanes of token rows past the expert's segment
//     get an offset past the buffer's range and read zeros without a memory
//     access.
// ---------------------------------------------------------------------------
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kStages = 3;
constexpr int kRowBytes = 128;                           // K bytes per row per step
constexpr int kScaleRegion = (kBM + kBN) * kRowBytes;    // fp8 token scales of the step
constexpr int kStageBytes = kScaleRegion + kBM * 4;      // 48 KB + 512 B
constexpr int kWRegion = kBM * kRowBytes;                // weight rows start here
constexpr int kDmaPerWave = (kBM + kBN) / 8 / 4;         // 12 loads of 8 rows per wave

// Buffer ranges are capped below kOobOffset, so a lane offset of kOobOffset
// is out of range: the load returns zeros without touching memory (used for
// token rows past the expert's segment).
constexpr int kBufMax = 0x7ffffe00;
constexpr int kOobOffset = 0x7fffff00;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > kBufMax ? kBufMax : (bytes < 0 ? 0 : static_cast<int>(bytes));
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

// Raises a kernel's dynamic-LDS limit to `bytes` once per device (the
// attribute belongs to the current device; `set` records the devices done).
// A failure is left to the launch to report.
inline void allow_dynamic_lds(const void* kern, int bytes, std::atomic<uint64_t>& set) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return;
  }
  const uint64_t bit = uint64_t(1) << dev;
  if (set.load(std::memory_order_acquire) & bit) return;
  if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
    (void)hipGetLastError();
  set.fetch_or(bit, std::memory_order_acq_rel);
}

template <bool FP8, int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_pipelined_kernel(const GemmArgs g) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  __shared__ float row_amax[2][kBM];
  constexpr bool kSwiglu = MODE == MODE_SWIGLU || MODE == MODE_SWIGLU_FP8OUT;
  constexpr int kKK = FP8 ? 2 : 4;             // MFMA sub-steps per K step
  // Direct loads per wave and step: 12 x 8 rows of operands, plus (fp8) one
  // 4-byte-per-lane load of token scales.  Every load that the step waits
  // count tracks is a direct load, so they retire in issue order.
  constexpr int kDmaStep = kDmaPerWave + (FP8 ? 1 : 0);

  const int total = *g.n_tiles * g.nt_n;
  const int per_xcd = ceil_div(total, kXcds);
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int t = (blockIdx.x % kXcds) * per_xcd + slot;
  if (t >= total) return;
  const int4 inf = g.info[t / g.nt_n];
  const int e = inf.x, u = t - inf.y * g.nt_n;
  const int nt = u / inf.z, mt = u % inf.z;
  const int2 sg = segment(g.seg, g.seg_cap, e);
  const int seg_end = sg.y;
  const int row0 = sg.x + mt * kBM;

  const int ldb = FP8 ? g.K : 2 * g.K;  // bytes per row of A and W
  const int nk = ldb / kRowBytes;
  // Buffer views advance by one K step at a time.  With a fused gather the
  // view spans the whole source and each lane's offset names its row.
  const int64_t a_skip = g.a_index ? 0 : static_cast<int64_t>(row0) * g.a_rs;
  const uint8_t* a_base = g.A + a_skip;
  const int64_t a_left = g.a_bytes - a_skip;
  const uint8_t* w_base = g.W + e * g.w_stride;

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
    // 16-byte chunk c of the step's 128 bytes is in 64-byte piece c / 4
    // (piece strides fit 32 bits: the host checks 64 N_cap < 2^31).
    const int cs = static_cast<int>(rr < kBM ? g.a_cs : g.w_cs);
    const int arow = rr < kBM && g.a_index && row0 + rr < seg_end ? g.a_index[row0 + rr] : rr;
    voff[q] = (rr < kBM ? arow * g.a_rs : grow * g.w_rs) + (chunk >> 2) * cs + (chunk & 3) * 16;
    if (rr < kBM && row0 + rr >= seg_end) voff[q] = kOobOffset;
    ldst[q] = grp * 1024;
  }
  // fp8: token scales of the step, 128 rows x 4 bytes, land beside the
  // operands (waves 0/1 and 2/3 load the same two halves; the duplicate
  // writes carry identical values).  With a fused gather the view spans
  // every source row's scales and each lane's offset names its row.
  const int kb_n = g.K / 128;
  const int srr = (w & 1) * 64 + lane;
  const __amdgpu_buffer_rsrc_t rS =
      !FP8        ? make_rsrc(g.A, 0)
      : g.a_index ? make_rsrc(g.A_scale, g.a_bytes / g.K * kb_n * 4)
                  : make_rsrc(g.A_scale + static_cast<int64_t>(row0) * kb_n,
                              static_cast<int64_t>(min(seg_end - row0, kBM)) * kb_n * 4);
  const int soffs = !g.a_index ? srr * kb_n * 4
                    : row0 + srr < seg_end ? g.a_index[row0 + srr] * kb_n * 4
                                           : kOobOffset;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(a_base, a_left);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(w_base, g.w_stride);
  auto dma = [&](int step, int stage) {
    const int k = min(step, nk - 1);  // step k starts at 64-byte K piece 2k
    uint8_t* base = smem + stage * kStageBytes;
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(q < 4 ? rA : rW, (lds_ptr_t)(base + ldst[q]), 16,
                                               voff[q], 2 * k * (q < 4 ? g.a_cs : g.w_cs), 0, 0);
    if (FP8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_ptr_t)(base + kScaleRegion + (w & 1) * 256),
                                               4, soffs, k * 4, 0, 0);
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

  // ---- fp8 scales: weight block scales are uniform per wave (scalar
  // loads); token group scales come from the stage in LDS.
  const float* swp[4];
  float sw[4], sx[2];
  if (FP8) {
    const int wnu = __builtin_amdgcn_readfirstlane(wn);
    const float* wsc = g.W_scale + e * g.ws_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lrow = wblock_row(kSwiglu, wnu, i);
      int grow;
      if (kSwiglu)
        grow = lrow < kBN / 2 ? nt * (kBN / 2) + lrow : g.Nout + nt * (kBN / 2) + (lrow - kBN / 2);
      else
        grow = min(nt * kBN + lrow, g.NW - 1);
      swp[i] = wsc + static_cast<int64_t>(grow / 128) * kb_n;
    }
  }
  auto load_wscales = [&](int step) {
    if (FP8) {
      // Through the constant address space: uniform loads become scalar
      // loads, which the step's vector-memory wait count does not see.
      const int k = min(step, nk - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sw[i] = ((const __attribute__((address_space(4))) float*)(uintptr_t)swp[i])[k];
    }
  };
  auto read_xscales = [&](const uint8_t* st) {
    if (FP8) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        sx[j] = *reinterpret_cast<const float*>(st + kScaleRegion + (wm * 64 + j * 32 + lr) * 4);
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

  // ---- prologue: steps 0, 1, 2 in flight
  dma(0, 0);
  dma(1, 1);
  dma(2, 2);
  load_wscales(0);
  WAIT_VMCNT(2 * kDmaStep);
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
    read_xscales(cur);
    mma(last, 0, 4);
    // Step boundary: this wave's loads of step kt+1 have landed once only
    // those of step kt+2 are in flight, and its own reads of stage kt are
    // done before anyone refills it.
    WAIT_VMCNT_LDS(kDmaStep);
    __builtin_amdgcn_s_barrier();
    // Stage kt is free in every wave now; refill it with step kt+3.
    lfrag(nxt, 0, 0);
    mma(last, 4, 4);
    if (FP8) {
      scale_acc();
      load_wscales(kt + 1);
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
  if constexpr (MODE == MODE_PLAIN || MODE == MODE_GELU) {
    uint8_t* C8 = static_cast<uint8_t*>(g.C);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = row0 + wm * 64 + j * 32 + lr;
      if (m >= seg_end) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nt * kBN + wn * 128 + i * 32 + q * 8 + cq;
          if (col >= g.Nout) continue;
          uint2 o;
          o.x = pack_bf16x2(plain_act<MODE>(acc[i][j][q * 4 + 0]), plain_act<MODE>(acc[i][j][q * 4 + 1]));
          o.y = pack_bf16x2(plain_act<MODE>(acc[i][j][q * 4 + 2]), plain_act<MODE>(acc[i][j][q * 4 + 3]));
          *reinterpret_cast<uint2*>(C8 + out_offset(g, m, col)) = o;
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
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint2 o;
            o.x = pack_bf16x2(acc[hb][j][q * 4 + 0], acc[hb][j][q * 4 + 1]);
            o.y = pack_bf16x2(acc[hb][j][q * 4 + 2], acc[hb][j][q * 4 + 3]);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(C) +
                                      out_offset(g, m, nt * 128 + wn * 64 + hb * 32 + q * 8 + cq)) = o;
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
  static_assert(kStages * kStageBytes + 2 * kBM * 4 <= 160 * 1024, "the ring fits the CU's LDS");
  auto kern = gemm_pipelined_kernel<FP8, MODE>;
  const size_t lds = kStages * kStageBytes;
  static std::atomic<uint64_t> lds_set{0};
  allow_dynamic_lds(reinterpret_cast<const void*>(kern), static_cast<int>(lds), lds_set);
  const int64_t blocks = (max_tiles * g.nt_n + kXcds - 1) / kXcds * kXcds + kXcds;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), lds, s, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Skinny bf16 kernel for a few rows per expert (decode): 32 token rows x 256
// weight rows per block, 4 waves each holding 32 x 64 (two MFMA 32x32 tiles;
// SwiGLU: the gate and up rows of the same 32 h columns).  The work is weight
// streaming, so the LDS goes to depth instead of token rows: four 36 KB
// stages of 128-byte K steps, loads three steps ahead (96 KB of weights in
// flight per CU).  Same addressing, gather and output layouts as the other
// kernels; rows past the segment load nothing.
// A block may have NW = 8 waves: waves 0-3 compute as above, and every wave
// issues its share of each step's direct loads (waves 4-7 only load and meet
// the barriers); sk_waves below says which element types use them.
// ---------------------------------------------------------------------------
constexpr int kSkBM = 32, kSkBN = 256;
// Cache policy of the skinny tiles' weight loads: non-temporal.  A decode
// FFN reads every active expert's weights once (GBs, far past the 256 MB
// MALL), so they need not stay in L2; the hint took the DeepSeek-V3 decode
// FFN from 396 to 372 us (bf16), 225 to 209 us (block-FP8) and 136 to
// 127 us (MXFP4).  Token and h rows keep the default policy: every n-tile
// of an m-tile reads them.
constexpr int kCpolStream = 2;
constexpr int kSkStages = 4;

// Tile t of a skinny GEMM (t < m-tiles x nt_n): the m-tile table entry holds
// the expert's first m-tile and m-tile count, and an expert's tiles run n-tile
// by n-tile, m-tile fastest.  Returns {expert, m-tile within the expert,
// n-tile, m-tile index in the table}.
__device__ __forceinline__ int4 skinny_decode(const GemmArgs& g, int t) {
  const int4 inf = g.info[t / g.nt_n];
  const int u = t - inf.y * g.nt_n;
  const int mt = u % inf.z;
  return make_int4(inf.x, mt, u / inf.z, inf.y + mt);
}

template <int MODE, int NW, int BN>
__device__ __forceinline__ void skinny_tile(const GemmArgs& g, int t, uint8_t* smem) {
  constexpr bool kSwiglu = MODE == MODE_SWIGLU || MODE == MODE_SWIGLU_FP8OUT;
  static_assert(BN == kSkBN || (NW == 8 && MODE == MODE_PLAIN && (BN == 384 || BN == 512)),
                "wider tiles: the plain (down) GEMM, eight waves");
  // ring: four 36 KB stages (256 weight rows), three of 52 KB (384) or two of
  // 68 KB (512)
  constexpr int kStg = BN == 256 ? kSkStages : BN == 384 ? 3 : 2;
  constexpr int kStageB = (kSkBM + BN) * kRowBytes;
  const int4 td = skinny_decode(g, t);
  const int e = td.x, mt = td.y, nt = td.z;
  const int2 sg = segment(g.seg, g.seg_cap, e);
  const int seg_end = sg.y;
  const int row0 = sg.x + mt * kSkBM;
  const int ldb = 2 * g.K;
  const int nk = ldb / kRowBytes;
  const int64_t a_skip = g.a_index ? 0 : static_cast<int64_t>(row0) * g.a_rs;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + a_skip, g.a_bytes - a_skip);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.W + e * g.w_stride, g.w_stride);
  const int nbase = kSwiglu ? nt * (kSkBN / 2) : nt * BN;

  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // direct loads: waves 0-3 move A group w (8 of the 32 rows); wave w moves
  // W groups 4 + kWPer w .. 4 + kWPer (w + 1) - 1
  constexpr int kWPer = BN / 8 / NW;
  const bool loads_a = w < kSkBM / 8, computes = w < BN / 64;
  const int wc = w & 3;                   // token row group
  const int wr = min(w, BN / 64 - 1);     // the compute role (offsets stay in range)
  // (sized for four waves: an array bound that depends on NW trips the host
  // pass's check of the 16-byte direct load)
  int voff[1 + kSkBN / 8 / 4], ldst[1 + kSkBN / 8 / 4];
#pragma unroll
  for (int q = 0; q < 1 + kWPer; ++q) {
    const int grp = q == 0 ? wc : kSkBM / 8 + w * kWPer + (q - 1);
    const int rr = grp * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((rr >> 1) & 7);
    if (rr < kSkBM) {
      const bool valid = row0 + rr < seg_end;
      const int arow = g.a_index && valid ? g.a_index[row0 + rr] : rr;
      voff[q] = valid ? arow * g.a_rs + (chunk >> 2) * g.a_cs + (chunk & 3) * 16 : kOobOffset;
    } else {
      const int r = rr - kSkBM;
      int grow;
      if (kSwiglu)
        grow = r < kSkBN / 2 ? min(nbase + r, g.Nout - 1)
                             : g.Nout + min(nbase + (r - kSkBN / 2), g.Nout - 1);
      else
        grow = min(nbase + r, g.NW - 1);
      voff[q] = grow * g.w_rs + (chunk >> 2) * g.w_cs + (chunk & 3) * 16;
    }
    ldst[q] = grp * 1024;
  }
  auto dma = [&](int step, int stage) {
    const int k = min(step, nk - 1);  // step k starts at 64-byte K piece 2k
    uint8_t* base = smem + stage * kStageB;
    if (loads_a)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(base + ldst[0]), 16, voff[0],
                                               2 * k * g.a_cs, 0, 0);
#pragma unroll
    for (int q = 1; q < 1 + kWPer; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_ptr_t)(base + ldst[q]), 16, voff[q],
                                               2 * k * g.w_cs, 0, kCpolStream);
  };
  // the wave's loads of kSkStages - 2 steps may stay in flight
  constexpr int kLa = (kStg - 2) * (1 + kWPer), kLw = (kStg - 2) * kWPer;

  const int lr = lane & 31, hi = lane >> 5, sl = (lr >> 1) & 7;
  int foff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) foff[kk] = lr * kRowBytes + (((2 * kk) | hi) ^ sl) * 16;
  int wbase[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    wbase[i] = (kSkBM + (kSwiglu ? i * (kSkBN / 2) + wr * 32 : wr * 64 + i * 32)) * kRowBytes;

  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

#pragma unroll
  for (int st = 0; st < kStg - 1; ++st) dma(st, st);
  if (loads_a)
    WAIT_VMCNT(kLa);
  else
    WAIT_VMCNT(kLw);
  __builtin_amdgcn_s_barrier();

  int s_cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const uint8_t* st = smem + s_cur * kStageB;
    dma(kt + kStg - 1, s_cur == 0 ? kStg - 1 : s_cur - 1);
    if (computes) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 fb = *reinterpret_cast<const bf16x8*>(st + foff[kk]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const bf16x8 fa = *reinterpret_cast<const bf16x8*>(st + wbase[i] + foff[kk]);
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc[i], 0, 0, 0);
        }
      }
    }
    if (loads_a)
      WAIT_VMCNT_LDS(kLa);
    else
      WAIT_VMCNT_LDS(kLw);
    __builtin_amdgcn_s_barrier();
    s_cur = s_cur + 1 == kStg ? 0 : s_cur + 1;
  }
  WAIT_VMCNT(0);
  if (!computes) return;  // the epilogue has no barrier

  // accumulator element q*4 + r: weight row q*8 + (lane/32)*4 + r of the
  // block, token row lane % 32
  const int cq = (lane >> 5) * 4;
  const int m = row0 + lr;
  if (m >= seg_end) return;
  uint8_t* C8 = static_cast<uint8_t*>(g.C);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (MODE == MODE_PLAIN || MODE == MODE_GELU) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int col = nbase + w * 64 + i * 32 + q * 8 + cq;
        if (col >= g.Nout) continue;
        uint2 o;
        o.x = pack_bf16x2(plain_act<MODE>(acc[i][q * 4 + 0]), plain_act<MODE>(acc[i][q * 4 + 1]));
        o.y = pack_bf16x2(plain_act<MODE>(acc[i][q * 4 + 2]), plain_act<MODE>(acc[i][q * 4 + 3]));
        *reinterpret_cast<uint2*>(C8 + out_offset(g, m, col)) = o;
      }
    } else {
      const int col = nbase + w * 32 + q * 8 + cq;
      if (col >= g.Nout) continue;
      float hv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = silu_mul(acc[0][q * 4 + r], acc[1][q * 4 + r]);
      uint2 o;
      o.x = pack_bf16x2(hv[0], hv[1]);
      o.y = pack_bf16x2(hv[2], hv[3]);
      *reinterpret_cast<uint2*>(C8 + out_offset(g, m, col)) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// Skinny block-FP8 tile for a few rows per expert (decode with block-FP8
// weights): the bf16 skinny tile's geometry -- 32 token rows x 256 weight
// rows, 4 waves of 32 x 64, four 36 KB stages three K steps ahead -- with
// 128-byte K steps of E4M3 (one 128-wide scale block each) and the
// pipelined FP8 kernel's arithmetic: a step's two MFMAs per 32 x 32 tile run
// into a zeroed temporary that is added to the sum times (weight block scale
// x token group scale).  Weight scales by scalar loads; the step's 32 token
// scales travel with the operands.  The up tile's 128 h columns are one
// quantisation group: the four waves exchange their row maxima in LDS and
// write E4M3 codes and the group scale amax / 448.  Both skinny tiles also
// come BN = 384 or 512 weight rows wide for the plain (down) GEMM: BN / 64
// computing waves of eight, three 52 KB or two 68 KB stages.
// ---------------------------------------------------------------------------

template <int MODE, int NW, int BN>
__device__ __forceinline__ void f8_skinny_tile(const GemmArgs& g, int t, uint8_t* smem) {
  constexpr bool kSwiglu = MODE == MODE_SWIGLU_FP8OUT;
  static_assert(BN == kSkBN || (NW == 8 && MODE == MODE_PLAIN && (BN == 384 || BN == 512)),
                "wider tiles: the plain (down) GEMM, eight waves");
  constexpr int kStg = BN == 256 ? kSkStages : BN == 384 ? 3 : 2;
  constexpr int kScaleOff = (kSkBM + BN) * kRowBytes;   // token scales after the rows
  constexpr int kStageB = kScaleOff + 256;
  __shared__ float row_amax[4][kSkBM];
  const int4 td = skinny_decode(g, t);
  const int e = td.x, mt = td.y, nt = td.z;
  const int2 sg = segment(g.seg, g.seg_cap, e);
  const int seg_end = sg.y;
  const int row0 = sg.x + mt * kSkBM;
  const int nk = g.K / kRowBytes;  // one E4M3 byte per element
  const int kb_n = g.K / 128;      // scale blocks per row
  // with a fused gather (a_index) the views span the whole source and each
  // lane's offset names its row
  const int64_t a_skip = g.a_index ? 0 : static_cast<int64_t>(row0) * g.a_rs;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + a_skip, g.a_bytes - a_skip);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.W + e * g.w_stride, g.w_stride);
  const __amdgpu_buffer_rsrc_t rS =
      g.a_index ? make_rsrc(g.A_scale, g.a_bytes / g.K * kb_n * 4)
                : make_rsrc(g.A_scale + static_cast<int64_t>(row0) * kb_n,
                            static_cast<int64_t>(min(seg_end - row0, kSkBM)) * kb_n * 4);
  const int nbase = kSwiglu ? nt * (kSkBN / 2) : nt * BN;

  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // direct loads: waves 0-3 move A group w (8 of the 32 rows), wave w W
  // groups 4 + kWPer w .. 4 + kWPer (w + 1) - 1, and every wave the step's
  // 32 token scales (the same values to the same place)
  constexpr int kWPer = BN / 8 / NW;
  const bool loads_a = w < kSkBM / 8, computes = w < BN / 64;
  const int wc = w & 3;                   // token row group
  const int wr = min(w, BN / 64 - 1);     // the compute role (offsets stay in range)
  // (sized for four waves: an array bound that depends on NW trips the host
  // pass's check of the 16-byte direct load)
  int voff[1 + kSkBN / 8 / 4], ldst[1 + kSkBN / 8 / 4];
#pragma unroll
  for (int q = 0; q < 1 + kWPer; ++q) {
    const int grp = q == 0 ? wc : kSkBM / 8 + w * kWPer + (q - 1);
    const int rr = grp * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((rr >> 1) & 7);
    if (rr < kSkBM) {
      const bool valid = row0 + rr < seg_end;
      const int arow = g.a_index && valid ? g.a_index[row0 + rr] : rr;
      voff[q] = valid ? arow * g.a_rs + chunk * 16 : kOobOffset;
    } else {
      const int r = rr - kSkBM;
      int grow;
      if (kSwiglu)
        grow = r < kSkBN / 2 ? min(nbase + r, g.Nout - 1)
                             : g.Nout + min(nbase + (r - kSkBN / 2), g.Nout - 1);
      else
        grow = min(nbase + r, g.NW - 1);
      voff[q] = grow * g.w_rs + chunk * 16;
    }
    ldst[q] = grp * 1024;
  }
  int soff = lane < kSkBM ? lane * kb_n * 4 : kOobOffset;
  if (g.a_index && lane < kSkBM)
    soff = row0 + lane < seg_end ? g.a_index[row0 + lane] * kb_n * 4 : kOobOffset;
  auto dma = [&](int step, int stage) {
    // steps past the last one load nothing (out-of-range offsets)
    const bool live = step < nk;
    const int k = live ? step : 0;
    uint8_t* base = smem + stage * kStageB;
    if (loads_a)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(base + ldst[0]), 16,
                                               live ? voff[0] : kOobOffset, k * kRowBytes, 0, 0);
#pragma unroll
    for (int q = 1; q < 1 + kWPer; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_ptr_t)(base + ldst[q]), 16,
                                               live ? voff[q] : kOobOffset, k * kRowBytes, 0,
                                               kCpolStream);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_ptr_t)(base + kScaleOff), 4,
                                             live ? soff : kOobOffset, k * 4, 0, 0);
  };
  // the wave's loads of kSkStages - 2 steps may stay in flight
  constexpr int kLa = (kStg - 2) * (2 + kWPer), kLw = (kStg - 2) * (1 + kWPer);

  // fragments: a lane holds 32 contiguous K bytes, [64 kk + 32 hi, +32), of
  // its row (chunks c and c ^ 1 after the swizzle); weight tiles i = 0, 1
  // (SwiGLU: gate rows w*32.., up rows 128 + w*32..; plain: w*64 + i*32..)
  const int lr = lane & 31, hi = lane >> 5, sl = (lr >> 1) & 7;
  int foff[4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int c0 = (4 * kk + 2 * hi) ^ sl;
    foff[2 * kk] = lr * kRowBytes + c0 * 16;
    foff[2 * kk + 1] = lr * kRowBytes + (c0 ^ 1) * 16;
  }
  int wbase[2];
  const float* swp[2];
  const float* wsc = g.W_scale + e * g.ws_stride;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int lrow = kSwiglu ? i * (kSkBN / 2) + wr * 32 : wr * 64 + i * 32;
    wbase[i] = (kSkBM + lrow) * kRowBytes;
    int grow;
    if (kSwiglu)
      grow = lrow < kSkBN / 2 ? nbase + lrow : g.Nout + nbase + (lrow - kSkBN / 2);
    else
      grow = min(nbase + lrow, g.NW - 1);
    swp[i] = wsc + static_cast<int64_t>(grow / 128) * kb_n;
  }

  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

#pragma unroll
  for (int st = 0; st < kStg - 1; ++st) dma(st, st);
  if (loads_a)
    WAIT_VMCNT(kLa);
  else
    WAIT_VMCNT(kLw);
  __builtin_amdgcn_s_barrier();

  int s_cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const uint8_t* st = smem + s_cur * kStageB;
    dma(kt + kStg - 1, s_cur == 0 ? kStg - 1 : s_cur - 1);
    if (computes) {
      // weight block scales through the constant address space (scalar loads,
      // outside the vector-memory wait count)
      float sw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        sw[i] = ((const __attribute__((address_space(4))) float*)(uintptr_t)swp[i])[kt];
      const float sx = *reinterpret_cast<const float*>(st + kScaleOff + lr * 4);
      f32x16 tmp[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmp[i][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const i32x4 b0 = *reinterpret_cast<const i32x4*>(st + foff[2 * kk]);
        const i32x4 b1 = *reinterpret_cast<const i32x4*>(st + foff[2 * kk + 1]);
        const i32x8 fb = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const i32x4 a0 = *reinterpret_cast<const i32x4*>(st + wbase[i] + foff[2 * kk]);
          const i32x4 a1 = *reinterpret_cast<const i32x4*>(st + wbase[i] + foff[2 * kk + 1]);
          const i32x8 fa = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          tmp[i] =
              __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, tmp[i], 0, 0, 0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float sc = sw[i] * sx;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] += tmp[i][r] * sc;
      }
    }
    if (loads_a)
      WAIT_VMCNT_LDS(kLa);
    else
      WAIT_VMCNT_LDS(kLw);
    __builtin_amdgcn_s_barrier();
    s_cur = s_cur + 1 == kStg ? 0 : s_cur + 1;
  }
  WAIT_VMCNT(0);

  // accumulator element q*4 + r: weight row q*8 + (lane/32)*4 + r of the
  // tile, token row lane % 32
  const int cq = hi * 4;
  const int m = row0 + lr;
  if constexpr (MODE == MODE_PLAIN) {
    if (!computes || m >= seg_end) return;
    uint8_t* C8 = static_cast<uint8_t*>(g.C);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = nbase + w * 64 + i * 32 + q * 8 + cq;
        if (col >= g.Nout) continue;
        uint2 o;
        o.x = pack_bf16x2(acc[i][q * 4 + 0], acc[i][q * 4 + 1]);
        o.y = pack_bf16x2(acc[i][q * 4 + 2], acc[i][q * 4 + 3]);
        *reinterpret_cast<uint2*>(C8 + out_offset(g, m, col)) = o;
      }
  } else {
    // h = silu(gate) * up; the tile's 128 h columns of a token (32 per wave)
    // are one group: row maxima over the four waves through LDS
    float hv[16];
    float am = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      hv[r] = silu_mul(acc[0][r], acc[1][r]);
      am = fmaxf(am, fabsf(hv[r]));
    }
    am = fmaxf(am, __shfl_xor(am, 32));
    if (computes && lane < 32) row_amax[w][lr] = am;
    __syncthreads();  // every wave of the block meets it
    am = fmaxf(fmaxf(row_amax[0][lr], row_amax[1][lr]), fmaxf(row_amax[2][lr], row_amax[3][lr]));
    const float sc = am > 0.0f ? am / 448.0f : 1.0f;
    if (!computes || m >= seg_end) return;
    uint8_t* crow = static_cast<uint8_t*>(g.C) + static_cast<int64_t>(m) * g.Nout;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* v = hv + q * 4;
      *reinterpret_cast<uint32_t*>(crow + nbase + w * 32 + q * 8 + cq) =
          f32x4_to_e4m3x4(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
    }
    if (w == 0 && lane < 32) g.C_scale[static_cast<int64_t>(m) * (g.Nout / 128) + nt] = sc;
  }
}

// ---------------------------------------------------------------------------
// MXFP4 weights x MXFP8 activations (OCP MX formats: E2M1 and E4M3 elements,
// one E8M0 scale 2^(e - 127) per 32 consecutive K elements of a row) on the
// block-scaled matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4, which
// applies both operands' scales inside the matrix core: no promotion step.
// Operand placement of one 32 x 32 x 64 instruction (measured on gfx950):
//   weights (A, E2M1): lane l holds weight row l % 32 and K [32 (l/32), +32),
//     16 bytes, low nibble first, and the E8M0 scale of that block;
//   tokens (B, E4M3): lane l holds token l % 32 and K [16 (l/32), +16) and
//     [32 + 16 (l/32), +16), and the E8M0 scale of block l / 32.
// Block tile 128 tokens x 256 weight rows, 4 waves of 64 x 128 (2 x 4 tiles,
// SwiGLU: the gate and up rows of the same 64 h columns); K steps of 128
// (64 bytes of E2M1 and 128 of E4M3 per row, 4 scale bytes each) through a
// four-stage LDS ring fed three steps ahead by direct-to-LDS loads.  The up
// GEMM's epilogue writes h as MXFP8: each 32-column block of one token is one
// instruction tile, split over lanes l and l ^ 32.
// ---------------------------------------------------------------------------
constexpr int kMxBN = 256;
constexpr int kMxK = 128;                                  // K elements per step

// Two block shapes: 128 token rows with 4 waves and a four-stage ring, or
// (many rows per expert) 256 token rows with 8 waves (two per SIMD) and three
// 50 KB stages.  A stage holds the token rows [BM][128 B], the weight rows
// [256][64 B], then one scale dword per token row and per weight row.
template <int BM_>
struct MxShape {
  static constexpr int BM = BM_, NW = BM / 64 * 2, THREADS = NW * 64;
  static constexpr int STAGES = BM == 128 ? 4 : 3;
  static constexpr int WOFF = BM * kMxK;
  static constexpr int SAOFF = WOFF + kMxBN * (kMxK / 2);
  static constexpr int SWOFF = SAOFF + BM * 4;
  static constexpr int STAGE_BYTES = SWOFF + kMxBN * 4;
  // direct loads per wave and step: token row groups (8 rows of 128 B),
  // weight row groups (16 rows of 64 B), scale dwords
  static constexpr int TL = BM / 8 / NW, WL = kMxBN / 16 / NW;
  static constexpr int LOADS = TL + WL + (BM == 128 ? 2 : 1);
  static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "the ring fits the CU's LDS");
};

// Unit u of an expert's tiles (tiles m-tiles, nt_n n-tiles) in L2-friendly
// order: groups of kMxGroup m-tiles, n-tile by n-tile within a group, m-tile
// fastest.  An XCD runs 32 consecutive units at once; one K step of an MX
// unit reads 32 KB of token rows (BM = 256) and 16 KB of weight rows, so
// 4 m-tiles x 8 n-tiles read 256 KB of distinct operand bytes per step where
// m-tile-fastest order over ~10 m-tiles x 3 n-tiles read 368 KB (the L2
// hit rate of its operand loads measured 72 %).  DeepSeek-V3 shard with
// MXFP4 weights: FFN 4.90 -> 4.52 ms (groups of 2 and 8: 4.59, 4.58).
constexpr int kMxGroup = 4;
__device__ __forceinline__ void mx_unit(int u, int tiles, int nt_n, int& mt, int& nt) {
  const int grp = u / (kMxGroup * nt_n);
  const int rem = u - grp * kMxGroup * nt_n;
  const int gs = min(kMxGroup, tiles - grp * kMxGroup);
  nt = rem / gs;
  mt = grp * kMxGroup + rem % gs;
}

// E8M0 exponent (biased) of a block whose largest magnitude is amax, for an
// element format whose largest normal has exponent emax: floor(log2 amax) -
// emax, clamped to the scale's range (an all-zero block takes 2^-127).
__device__ __forceinline__ int mx_scale_code(float amax, int emax) {
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff);
  if (e == 0) return 0;                       // zero or subnormal: at or below 2^-127
  const int s = e - 127 - emax;
  return (s < -127 ? -127 : s) + 127;
}

template <int MODE, class SH>
__device__ __forceinline__ void mx_tile(const GemmArgs& g, uint8_t* smem) {
  constexpr bool kSwiglu = MODE == MODE_SWIGLU_MX8OUT;
  constexpr int kMxBM = SH::BM, kMxStages = SH::STAGES, kMxStageBytes = SH::STAGE_BYTES;
  constexpr int kMxWOff = SH::WOFF, kMxSAOff = SH::SAOFF, kMxSWOff = SH::SWOFF;
  constexpr int kMxLoads = SH::LOADS, TL = SH::TL, WL = SH::WL;
  const int total = *g.n_tiles * g.nt_n;
  const int per_xcd = ceil_div(total, kXcds);
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int t = (blockIdx.x % kXcds) * per_xcd + slot;
  if (t >= total) return;
  const int4 inf = g.info[t / g.nt_n];
  const int e = inf.x, u = t - inf.y * g.nt_n;
  int mt, nt;
  mx_unit(u, inf.z, g.nt_n, mt, nt);
  const int2 sg = segment(g.seg, g.seg_cap, e);
  const int seg_end = sg.y;
  const int row0 = sg.x + mt * kMxBM;
  const int K = g.K, kb = K / 32;                 // scale bytes per row
  const int nk = K / kMxK;
  const uint8_t* As = reinterpret_cast<const uint8_t*>(g.A_scale);
  const uint8_t* Ws = reinterpret_cast<const uint8_t*>(g.W_scale);
  // with a fused gather (a_index) the token views span the whole source and
  // each lane's offset names its row (arow: valid rows only)
  const int64_t a_skip = g.a_index ? 0 : static_cast<int64_t>(row0) * K;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + a_skip, g.a_bytes - a_skip);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.W + e * g.w_stride, g.w_stride);
  const __amdgpu_buffer_rsrc_t rAS =
      make_rsrc(As + a_skip / K * kb, (g.a_bytes - a_skip) / K * kb);
  const __amdgpu_buffer_rsrc_t rWS = make_rsrc(Ws + e * g.ws_stride, g.ws_stride);
  const int nbase = kSwiglu ? nt * (kMxBN / 2) : nt * kMxBN;
  auto arow = [&](int rr) { return g.a_index ? g.a_index[row0 + rr] : rr; };
  auto wrow = [&](int r) {  // weight row (within the expert) of tile row r
    if (kSwiglu)
      return r < kMxBN / 2 ? min(nbase + r, g.Nout - 1)
                           : g.Nout + min(nbase + (r - kMxBN / 2), g.Nout - 1);
    return min(nbase + r, g.NW - 1);
  };

  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  // Direct loads of wave w per step: token row groups TL w.., weight row
  // groups WL w.., and scale dwords (a direct load writes one dword per lane,
  // so scales move as whole dwords).  128 rows: 64 weight scales (rows 64w..)
  // and 64 token scales (rows 64 (w & 1)..; waves w and w ^ 2 write the same
  // values to the same place).  256 rows: waves 0-3 the token scales of rows
  // 64w.., waves 4-7 the weight scales of rows 64 (w - 4)...
  int voff[kMxLoads];
#pragma unroll
  for (int q = 0; q < TL; ++q) {
    const int rr = (w * TL + q) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((rr >> 1) & 7);
    voff[q] = row0 + rr < seg_end ? arow(rr) * K + c * 16 : kOobOffset;
  }
#pragma unroll
  for (int q = 0; q < WL; ++q) {
    const int r = (w * WL + q) * 16 + (lane >> 2);
    const int cw = (lane & 3) ^ ((r >> 2) & 3);
    voff[TL + q] = wrow(r) * g.w_rs + cw * 16;
  }
  bool s_tok;      // 256 rows: this wave's scale load is a token-scale one
  int s_lds;
  if constexpr (kMxBM == 128) {
    voff[TL + WL] = wrow(w * 64 + lane) * g.ws_rs;
    const int rr = (w & 1) * 64 + lane;
    voff[TL + WL + 1] = row0 + rr < seg_end ? arow(rr) * kb : kOobOffset;
    s_tok = false;
    s_lds = 0;
  } else {
    s_tok = w < 4;
    if (s_tok) {
      const int rr = w * 64 + lane;
      voff[TL + WL] = row0 + rr < seg_end ? arow(rr) * kb : kOobOffset;
      s_lds = kMxSAOff + w * 256;
    } else {
      voff[TL + WL] = wrow((w - 4) * 64 + lane) * g.ws_rs;
      s_lds = kMxSWOff + (w - 4) * 256;
    }
  }
  auto dma = [&](int step, int stage) {
    // steps past the last one load nothing (out-of-range offsets)
    const bool live = step < nk;
    const int k = live ? step : 0;
    uint8_t* base = smem + stage * kMxStageBytes;
#pragma unroll
    for (int q = 0; q < TL; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(base + (w * TL + q) * 1024), 16,
                                               live ? voff[q] : kOobOffset, k * kMxK, 0, 0);
#pragma unroll
    for (int q = 0; q < WL; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_ptr_t)(base + kMxWOff + (w * WL + q) * 1024),
                                               16, live ? voff[TL + q] : kOobOffset, k * g.w_cs, 0,
                                               0);
    if constexpr (kMxBM == 128) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rWS, (lds_ptr_t)(base + kMxSWOff + w * 256), 4,
                                               live ? voff[TL + WL] : kOobOffset, k * g.ws_cs, 0,
                                               0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rAS, (lds_ptr_t)(base + kMxSAOff + (w & 1) * 256),
                                               4, live ? voff[TL + WL + 1] : kOobOffset, k * 4, 0,
                                               0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_tok ? rAS : rWS, (lds_ptr_t)(base + s_lds), 4,
                                               live ? voff[TL + WL] : kOobOffset,
                                               k * (s_tok ? 4 : g.ws_cs), 0, 0);
    }
  };

  // Fragment addresses: wave (wm, wn) holds tokens wm*64.. and weight rows
  // wblock_row(i) + (lane % 32) for its four weight tiles.
  const int wm = w >> 1, wn = w & 1;
  const int lr = lane & 31, hi = lane >> 5;
  int wfr[4][2], wsc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wblock_row(kSwiglu, wn, i) + lr;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      wfr[i][hh] = kMxWOff + r * 64 + (((2 * hh + hi) ^ ((r >> 2) & 3)) * 16);
    wsc[i] = kMxSWOff + r * 4;
  }
  int tfr[2][2][2], tsc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rr = wm * 64 + j * 32 + lr;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      tfr[j][hh][0] = rr * kMxK + (((4 * hh + hi) ^ ((rr >> 1) & 7)) * 16);
      tfr[j][hh][1] = rr * kMxK + (((4 * hh + 2 + hi) ^ ((rr >> 1) & 7)) * 16);
    }
    tsc[j] = kMxSAOff + rr * 4;
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
  for (int st = 0; st < kMxStages - 1; ++st) dma(st, st);
  WAIT_VMCNT((kMxStages - 2) * kMxLoads);
  __builtin_amdgcn_s_barrier();

  int s_cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const uint8_t* st = smem + s_cur * kMxStageBytes;
    dma(kt + kMxStages - 1, s_cur == 0 ? kMxStages - 1 : s_cur - 1);
    uint32_t ws[4], ts[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) ws[i] = *reinterpret_cast<const uint32_t*>(st + wsc[i]);
#pragma unroll
    for (int j = 0; j < 2; ++j) ts[j] = *reinterpret_cast<const uint32_t*>(st + tsc[j]);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      i32x8 tb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const i32x4 p0 = *reinterpret_cast<const i32x4*>(st + tfr[j][hh][0]);
        const i32x4 p1 = *reinterpret_cast<const i32x4*>(st + tfr[j][hh][1]);
        tb[j] = i32x8{p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x4 p = *reinterpret_cast<const i32x4*>(st + wfr[i][hh]);
        const i32x8 wa = i32x8{p[0], p[1], p[2], p[3], 0, 0, 0, 0};
        const int sa = static_cast<int>((ws[i] >> (16 * hh + 8 * hi)) & 0xff);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int sb = static_cast<int>((ts[j] >> (16 * hh + 8 * hi)) & 0xff);
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa, tb[j], acc[i][j], 4, 0,
                                                                       0, sa, 0, sb);
        }
      }
    }
    WAIT_VMCNT_LDS((kMxStages - 2) * kMxLoads);
    __builtin_amdgcn_s_barrier();
    s_cur = s_cur + 1 == kMxStages ? 0 : s_cur + 1;
  }
  WAIT_VMCNT(0);

  // accumulator element q*4 + r: weight row q*8 + (lane/32)*4 + r of the
  // tile, token lane % 32
  const int cq = hi * 4;
  uint8_t* C8 = static_cast<uint8_t*>(g.C);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = row0 + wm * 64 + j * 32 + lr;
    const bool live = m < seg_end;
    if constexpr (MODE == MODE_PLAIN) {
      if (!live) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nbase + wn * 128 + i * 32 + q * 8 + cq;
          if (col >= g.Nout) continue;
          uint2 o;
          o.x = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
          o.y = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
          *reinterpret_cast<uint2*>(C8 + (static_cast<int64_t>(m) * g.Nout + col) * 2) = o;
        }
    } else {
      // h = silu(gate) * up; one 32-column MX block per (i, token), held by
      // lanes l and l ^ 32 (shuffles run in every lane, live or not)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float hv[16];
        float amax = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          hv[r] = silu_mul(acc[i][j][r], acc[i + 2][j][r]);
          amax = fmaxf(amax, fabsf(hv[r]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const int code = mx_scale_code(amax, 8);
        const int c0 = nbase + wn * 64 + i * 32;   // first h column of the block
        if (!live || c0 >= g.Nout) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float* v = hv + q * 4;
          const uint32_t p = f32x4_to_e4m3x4(ldexpf(v[0], 127 - code), ldexpf(v[1], 127 - code),
                                             ldexpf(v[2], 127 - code), ldexpf(v[3], 127 - code));
          *reinterpret_cast<uint32_t*>(C8 + static_cast<int64_t>(m) * g.Nout + c0 + q * 8 + cq) = p;
        }
        if (hi == 0) reinterpret_cast<uint8_t*>(g.C_scale)[static_cast<int64_t>(m) * (g.Nout / 32) + c0 / 32] =
            static_cast<uint8_t>(code);
      }
    }
  }
}

template <int MODE, int BM>
__global__ __launch_bounds__(MxShape<BM>::THREADS, 1) void gemm_mx_kernel(const GemmArgs g) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  mx_tile<MODE, MxShape<BM>>(g, smem);
}

template <int MODE, int BM>
hipError_t launch_mx(const GemmArgs& g, int64_t max_tiles, hipStream_t s) {
  using SH = MxShape<BM>;
  auto kern = gemm_mx_kernel<MODE, BM>;
  const size_t lds = SH::STAGES * SH::STAGE_BYTES;
  static std::atomic<uint64_t> lds_set{0};
  allow_dynamic_lds(reinterpret_cast<const void*>(kern), static_cast<int>(lds), lds_set);
  const int64_t blocks = (max_tiles * g.nt_n + kXcds - 1) / kXcds * kXcds + kXcds;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(SH::THREADS), lds, s, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Skinny MX kernel for a few rows per expert (decode with MXFP4 weights):
// 32 token rows x 256 weight rows per block, 4 waves each holding 32 x 64
// (two 32 x 32 instruction tiles; SwiGLU: the gate and up rows of the same
// 32 h columns, i.e. one MX block of h per token).  As in the bf16 skinny
// kernel the work is weight streaming and the LDS goes to depth: K steps of
// 128 (64 bytes of E2M1 per weight row, 16 KB per step) through a seven-stage
// ring of 21 KB stages, loads six steps ahead (96 KB of weights in flight per
// CU).  Operand placement, swizzles and the MXFP8 h epilogue are those of the
// 128-row MX tile.  A stage holds the token rows [32][128 B], the weight rows
// [256][64 B], 64 token-scale dwords (rows 32..63 read as zeros) and 256
// weight-scale dwords.
// ---------------------------------------------------------------------------
constexpr int kMsBM = 32;
// Ring of the skinny MX tile with BN weight rows: a stage holds the token
// rows [32][128 B], the weight rows [BN][64 B], 64 token-scale dwords and BN
// weight-scale dwords; seven stages of 21 KB (BN = 256) or four of 38 KB
// (BN = 512, the down GEMM's tile: half the tiles, so half the per-tile
// costs -- ticket, table reads, first loads, the acquire that invalidates the
// XCD's L2 -- for the same weight bytes in flight).
template <int BN> struct MsGeom {
  static constexpr int kWOff = kMsBM * kMxK;               // 4 KB of token rows
  static constexpr int kTSOff = kWOff + BN * (kMxK / 2);   // weight rows
  static constexpr int kWSOff = kTSOff + 64 * 4;           // token scales
  static constexpr int kStageBytes = kWSOff + BN * 4;      // weight scales
  static constexpr int kStages = BN == 256 ? 7 : 4;
  static_assert(kStages * kStageBytes <= 160 * 1024 - 1024, "the ring fits the CU's LDS");
};
constexpr size_t kMsRingBytes =
    MsGeom<256>::kStages * MsGeom<256>::kStageBytes > MsGeom<512>::kStages * MsGeom<512>::kStageBytes
        ? MsGeom<256>::kStages * MsGeom<256>::kStageBytes
        : MsGeom<512>::kStages * MsGeom<512>::kStageBytes;
// A step's loads: 4 token row groups (8 rows), BN / 16 weight row groups (16
// rows), BN / 64 weight-scale loads (64 rows) and the token scales, which
// every wave loads (the same values to the same place).  BN = 256, 4 waves:
// a wave takes one of each and 4 weight groups (7 loads); 8 waves: 2 weight
// groups and a token group (waves 0-3) or a weight-scale load (waves 4-7)
// (4 loads).  BN = 512, 8 waves: 4 weight groups, a weight-scale load and a
// token group (waves 0-3: 7 loads, the others 6).

template <int MODE, int NW, int BN>
__device__ __forceinline__ void mx_skinny_tile(const GemmArgs& g, int t, uint8_t* smem) {
  constexpr bool kSwiglu = MODE == MODE_SWIGLU_MX8OUT;
  static_assert(BN == 256 || (BN == 512 && NW == 8 && MODE == MODE_PLAIN),
                "512-row tiles: the plain (down) GEMM, eight computing waves");
  using G = MsGeom<BN>;
  constexpr int kMsStages = G::kStages, kMsStageBytes = G::kStageBytes;
  constexpr int kMsWOff = G::kWOff, kMsTSOff = G::kTSOff, kMsWSOff = G::kWSOff;
  const int4 td = skinny_decode(g, t);
  const int e = td.x, mt = td.y, nt = td.z;
  const int2 sg = segment(g.seg, g.seg_cap, e);
  const int seg_end = sg.y;
  const int row0 = sg.x + mt * kMsBM;
  const int K = g.K, kb = K / 32, nk = K / kMxK;
  const uint8_t* As = reinterpret_cast<const uint8_t*>(g.A_scale);
  const uint8_t* Ws = reinterpret_cast<const uint8_t*>(g.W_scale);
  // with a fused gather (a_index) the token views span the whole source and
  // each lane's offset names its row (arow: valid rows only)
  const int64_t a_skip = g.a_index ? 0 : static_cast<int64_t>(row0) * K;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + a_skip, g.a_bytes - a_skip);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.W + e * g.w_stride, g.w_stride);
  const __amdgpu_buffer_rsrc_t rAS =
      make_rsrc(As + a_skip / K * kb, (g.a_bytes - a_skip) / K * kb);
  const __amdgpu_buffer_rsrc_t rWS = make_rsrc(Ws + e * g.ws_stride, g.ws_stride);
  const int nbase = kSwiglu ? nt * (kMxBN / 2) : nt * BN;
  auto arow = [&](int rr) { return g.a_index ? g.a_index[row0 + rr] : rr; };
  auto wrow = [&](int r) {  // weight row (within the expert) of tile row r
    if (kSwiglu)
      return r < kMxBN / 2 ? min(nbase + r, g.Nout - 1)
                           : g.Nout + min(nbase + (r - kMxBN / 2), g.Nout - 1);
    return min(nbase + r, g.NW - 1);
  };

  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int kWPer = BN / 16 / NW;  // weight row groups per wave
  const bool computes = BN == 512 || w < 4;
  const bool loads_a = NW == 4 || w < 4;
  const bool loads_ws = NW == 4 || BN == 512 || w >= 4;
  const int wc = w & 3;                                  // token row group
  const int wr = BN == 512 ? w : wc;                     // the compute role
  const int wsw = NW == 4 || BN == 512 ? w : w & 3;      // the weight-scale load's 64 rows
  int voff[16 / 4 + 3];  // sized for the largest count, 7 (see the bf16 tile)
  {
    const int rr = wc * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((rr >> 1) & 7);
    voff[0] = row0 + rr < seg_end ? arow(rr) * K + c * 16 : kOobOffset;
  }
#pragma unroll
  for (int q = 0; q < kWPer; ++q) {
    const int r = (w * kWPer + q) * 16 + (lane >> 2);
    const int cw = (lane & 3) ^ ((r >> 2) & 3);
    voff[1 + q] = wrow(r) * g.w_rs + cw * 16;
  }
  voff[kWPer + 1] = wrow(wsw * 64 + lane) * g.ws_rs;
  voff[kWPer + 2] = lane < kMsBM && row0 + lane < seg_end ? arow(lane) * kb : kOobOffset;
  auto dma = [&](int step, int stage) {
    // steps past the last one load nothing (out-of-range offsets)
    const bool live = step < nk;
    const int k = live ? step : 0;
    uint8_t* base = smem + stage * kMsStageBytes;
    if (loads_a)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(base + wc * 1024), 16,
                                               live ? voff[0] : kOobOffset, k * kMxK, 0, 0);
#pragma unroll
    for (int q = 0; q < kWPer; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rW, (lds_ptr_t)(base + kMsWOff + (w * kWPer + q) * 1024), 16,
          live ? voff[1 + q] : kOobOffset, k * g.w_cs, 0, kCpolStream);
    if (loads_ws)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rWS, (lds_ptr_t)(base + kMsWSOff + wsw * 256), 4,
                                               live ? voff[kWPer + 1] : kOobOffset, k * g.ws_cs,
                                               0, kCpolStream);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rAS, (lds_ptr_t)(base + kMsTSOff), 4,
                                             live ? voff[kWPer + 2] : kOobOffset, k * 4, 0, 0);
  };
  // the wave's loads of kMsStages - 2 steps may stay in flight
  constexpr int kWaitAll = (kMsStages - 2) * (kWPer + 3), kWaitOne = (kMsStages - 2) * (kWPer + 2);
  static_assert((kMsStages - 1) * (kWPer + 3) < 64, "loads in flight fit the vmcnt counter");
  const bool all_loads = loads_a && loads_ws;

  // fragments: weight tiles i = 0, 1 of wave w (SwiGLU: gate rows w*32.. and
  // up rows 128 + w*32..; plain: rows w*64 + i*32..), token lane % 32
  const int lr = lane & 31, hi = lane >> 5;
  int wfr[2][2], wsc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (kSwiglu ? i * (kMxBN / 2) + wr * 32 : wr * 64 + i * 32) + lr;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      wfr[i][hh] = kMsWOff + r * 64 + (((2 * hh + hi) ^ ((r >> 2) & 3)) * 16);
    wsc[i] = kMsWSOff + r * 4;
  }
  int tfr[2][2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    tfr[hh][0] = lr * kMxK + (((4 * hh + hi) ^ ((lr >> 1) & 7)) * 16);
    tfr[hh][1] = lr * kMxK + (((4 * hh + 2 + hi) ^ ((lr >> 1) & 7)) * 16);
  }
  const int tsc = kMsTSOff + lr * 4;

  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

#pragma unroll
  for (int st = 0; st < kMsStages - 1; ++st) dma(st, st);
  if (all_loads)
    WAIT_VMCNT(kWaitAll);
  else
    WAIT_VMCNT(kWaitOne);
  __builtin_amdgcn_s_barrier();

  int s_cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const uint8_t* st = smem + s_cur * kMsStageBytes;
    dma(kt + kMsStages - 1, s_cur == 0 ? kMsStages - 1 : s_cur - 1);
    if (computes) {
      const uint32_t ts = *reinterpret_cast<const uint32_t*>(st + tsc);
      uint32_t ws[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) ws[i] = *reinterpret_cast<const uint32_t*>(st + wsc[i]);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const i32x4 p0 = *reinterpret_cast<const i32x4*>(st + tfr[hh][0]);
        const i32x4 p1 = *reinterpret_cast<const i32x4*>(st + tfr[hh][1]);
        const i32x8 tb = i32x8{p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        const int sb = static_cast<int>((ts >> (16 * hh + 8 * hi)) & 0xff);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const i32x4 p = *reinterpret_cast<const i32x4*>(st + wfr[i][hh]);
          const i32x8 wa = i32x8{p[0], p[1], p[2], p[3], 0, 0, 0, 0};
          const int sa = static_cast<int>((ws[i] >> (16 * hh + 8 * hi)) & 0xff);
          acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa, tb, acc[i], 4, 0, 0, sa,
                                                                    0, sb);
        }
      }
    }
    if (all_loads)
      WAIT_VMCNT_LDS(kWaitAll);
    else
      WAIT_VMCNT_LDS(kWaitOne);
    __builtin_amdgcn_s_barrier();
    s_cur = s_cur + 1 == kMsStages ? 0 : s_cur + 1;
  }
  WAIT_VMCNT(0);
  if (!computes) return;  // the epilogue has no barrier

  // accumulator element q*4 + r: weight row q*8 + (lane/32)*4 + r of the
  // tile, token lane % 32
  const int cq = hi * 4;
  const int m = row0 + lr;
  const bool live = m < seg_end;
  uint8_t* C8 = static_cast<uint8_t*>(g.C);
  if constexpr (MODE == MODE_PLAIN) {
    if (!live) return;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = nbase + w * 64 + i * 32 + q * 8 + cq;
        if (col >= g.Nout) continue;
        uint2 o;
        o.x = pack_bf16x2(acc[i][q * 4 + 0], acc[i][q * 4 + 1]);
        o.y = pack_bf16x2(acc[i][q * 4 + 2], acc[i][q * 4 + 3]);
        *reinterpret_cast<uint2*>(C8 + (static_cast<int64_t>(m) * g.Nout + col) * 2) = o;
      }
  } else {
    // h = silu(gate) * up: the wave's 32 h columns of one token are one MX
    // block, held by lanes l and l ^ 32 (the shuffle runs in every lane)
    float hv[16];
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      hv[r] = silu_mul(acc[0][r], acc[1][r]);
      amax = fmaxf(amax, fabsf(hv[r]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const int code = mx_scale_code(amax, 8);
    const int c0 = nbase + w * 32;
    if (!live || c0 >= g.Nout) return;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* v = hv + q * 4;
      const uint32_t p = f32x4_to_e4m3x4(ldexpf(v[0], 127 - code), ldexpf(v[1], 127 - code),
                                         ldexpf(v[2], 127 - code), ldexpf(v[3], 127 - code));
      *reinterpret_cast<uint32_t*>(C8 + static_cast<int64_t>(m) * g.Nout + c0 + q * 8 + cq) = p;
    }
    if (hi == 0)
      reinterpret_cast<uint8_t*>(g.C_scale)[static_cast<int64_t>(m) * (g.Nout / 32) + c0 / 32] =
          static_cast<uint8_t>(code);
  }
}

// ---------------------------------------------------------------------------
// Both GEMMs of a decode-sized FFN in one launch.  Two launches leave each
// GEMM's last wave of tiles partly empty (448 up and 784 down tiles on 256
// CUs for the DeepSeek-V3 shard's decode batch: 1.75 and 3.06 waves) and
// leave a gap between them; here every block takes the next ticket of one
// queue -- all up tiles, then all down tiles -- so CUs freed by the up GEMM go
// straight on to down tiles and the weights stream without a break.
//  * An up tile stores its h columns, waits for its stores (workgroup-scope
//    release), meets at a block barrier, and one thread then releases at
//    device scope (which writes the XCD's L2 back) and adds one to its
//    m-tile's counter.
//  * A down tile's first thread polls its m-tile's counter until it equals
//    the number of up n-tiles and then acquires at device scope (which
//    invalidates the CU's and the XCD's caches) before the block barrier, so
//    the tile's h loads see the up tiles' stores.
//  One release per up tile and one acquire per down tile: with a device fence
//  in every thread the cache write-backs and invalidations cost the decode
//  FFN 35 % (0.548 against 0.403 ms for the DeepSeek-V3 decode batch).
// Tickets are taken in order and every up ticket precedes every down ticket,
// so a down tile waits only on up tiles that blocks already running hold,
// and up tiles wait on nothing: every wait ends.  The wait is still bounded:
// a down tile whose m-tile is not complete after spin_limit polls (which can
// only happen if that argument failed) sets kFlagWaitTimeout in the FFN's
// status word and skips its tile, so the kernel always ends and the caller
// learns that the output is incomplete.  wait_extra raises the count a down
// tile waits for (0 in normal use; a count no up tile can reach lets a test
// drive every down tile into the timeout with every kernel still ending).
// The grid has a block for every possible ticket; blocks whose ticket is past
// the live work return at once.
// ---------------------------------------------------------------------------
constexpr int kSpinLimit = 1 << 22;  // about half a second of s_sleep 2 polls

// KIND: the skinny tiles of one element type -- kSkBf16, kSkMx (MXFP4
// weights, MXFP8 tokens and h) or kSkFp8 (block-FP8).
enum { kSkBf16 = 0, kSkMx = 1, kSkFp8 = 2 };
// Waves per block of the skinny tiles of each element type (waves 0-3
// compute, the others only load).  Measured on the DeepSeek-V3 decode batch
// (FFN, 8 against 4 waves, alternating runs on one GPU): block-FP8 0.214 ->
// 0.211 ms, MXFP4 0.1345 -> 0.1336 ms, bf16 0.3778 -> 0.3789 ms; so the
// load stream of these tiles is not bound by the waves that issue it.
constexpr int sk_waves(int kind) { return kind == kSkBf16 ? 4 : 8; }
// Weight rows of the bf16 and block-FP8 down GEMM's skinny tile (the up
// GEMM's are 256).  Block-FP8 takes 384 (six computing waves, three 52 KB
// stages: the same 96 KB in flight, a third fewer down tiles): DeepSeek-V3
// decode FFN 0.2110 -> 0.2091 ms; 512 rows (two 68 KB stages, one step
// ahead) 0.2177 ms.  bf16: 384 rows 0.3776 -> 0.3823 ms, 512 rows 0.4045 ms.
constexpr int sk_down_bn(int kind) { return kind == kSkFp8 ? 384 : kSkBN; }
// LDS ring of a bf16 / block-FP8 skinny tile with bn weight rows.
constexpr size_t sk_ring(int bn, bool fp8) {
  return static_cast<size_t>(bn == 256 ? kSkStages : bn == 384 ? 3 : 2) *
         ((kSkBM + bn) * kRowBytes + (fp8 ? 256 : 0));
}
// Weight rows of the MX down GEMM's skinny tile (the up GEMM's are 256).
constexpr int kMsDownBN = 512;
template <int UPMODE, int KIND>
__global__ __launch_bounds__(64 * sk_waves(KIND), 1) void ffn_fused_skinny_kernel(
    const GemmArgs gu, const GemmArgs gd, int32_t* sync, int32_t* status, int wait_extra,
    int spin_limit) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  __shared__ int s_ticket, s_ready;
  const int n_m = *gu.n_tiles;  // live m-tiles (one table for both GEMMs)
  const int n_up = n_m * gu.nt_n, total = n_up + n_m * gd.nt_n;
  if (threadIdx.x == 0) s_ticket = atomicAdd(sync, 1);
  __syncthreads();
  const int t = s_ticket;
  if (t >= total) return;
  int32_t* done = sync + 1;
  constexpr int NW = sk_waves(KIND);
  if (t < n_up) {
    if constexpr (KIND == kSkMx)
      mx_skinny_tile<UPMODE, NW, 256>(gu, t, smem);
    else if constexpr (KIND == kSkFp8)
      f8_skinny_tile<UPMODE, NW, kSkBN>(gu, t, smem);
    else
      skinny_tile<UPMODE, NW, kSkBN>(gu, t, smem);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      atomicAdd(done + skinny_decode(gu, t).w, 1);
    }
    return;
  }
  const int td = t - n_up;
  if (threadIdx.x == 0) {
    const int32_t* c = done + skinny_decode(gd, td).w;
    const int need = gu.nt_n + wait_extra;
    int ready = 0;
    for (int it = 0;; ++it) {
      if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) {
        ready = 1;
        break;
      }
      if (it >= spin_limit) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (!ready) atomicOr(status, kFlagWaitTimeout);
    s_ready = ready;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!s_ready) return;  // reported through the status word
  if constexpr (KIND == kSkMx)
    mx_skinny_tile<MODE_PLAIN, NW, kMsDownBN>(gd, td, smem);
  else if constexpr (KIND == kSkFp8)
    f8_skinny_tile<MODE_PLAIN, NW, sk_down_bn(kSkFp8)>(gd, td, smem);
  else
    skinny_tile<MODE_PLAIN, NW, sk_down_bn(kSkBf16)>(gd, td, smem);
}

template <int UPMODE, int KIND>
hipError_t launch_fused(const GemmArgs& gu, const GemmArgs& gd, int64_t max_tiles, int32_t* sync,
                        int32_t* status, hipStream_t s) {
  static_assert(sk_ring(kSkBN, true) <= 160 * 1024 - 1024 &&
                    sk_ring(sk_down_bn(KIND), KIND == kSkFp8) <= 160 * 1024 - 1024,
                "the rings fit the CU's LDS");
  auto kern = ffn_fused_skinny_kernel<UPMODE, KIND>;
  const size_t lds = KIND == kSkMx    ? kMsRingBytes
                     : std::max(sk_ring(kSkBN, KIND == kSkFp8),
                                sk_ring(sk_down_bn(KIND), KIND == kSkFp8));
  static std::atomic<uint64_t> lds_set{0};
  allow_dynamic_lds(reinterpret_cast<const void*>(kern), static_cast<int>(lds), lds_set);
  const int64_t blocks = max_tiles * (gu.nt_n + gd.nt_n);
  // A test drives every down tile into the bounded wait's timeout by setting
  // MOE_TEST_FUSED_WAIT_UNREACHABLE=1: the down tiles then wait for one more
  // up tile than exists, for a few polls only (every kernel still ends).
  const char* unreachable = getenv("MOE_TEST_FUSED_WAIT_UNREACHABLE");
  const bool test_timeout = unreachable && unreachable[0] == '1';
  const int wait_extra = test_timeout ? 1 : 0;
  const int spin_limit = test_timeout ? 16 : kSpinLimit;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(64 * sk_waves(KIND)), lds, s,
                     gu, gd, sync, status, wait_extra, spin_limit);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Large-tile bf16 kernel, 8 waves (two per SIMD), each wave WM x 128 output
// elements (WM/32 x 4 MFMA 32x32 tiles).  Three block shapes share the code:
//   full tile: 256 token rows x 256 weight rows, waves 4 (rows) x 2 (weights)
//              of 64 x 128;
//   tall tile: 384 token rows x 256 weight rows, waves 4 x 2 of 96 x 128 --
//              the full tile of problems with many rows per expert;
//   wide tile: 128 token rows x 512 weight rows, waves 2 x 4 of 64 x 128 --
//              used for the last 1..128 rows of an expert's segment, which a
//              full or tall tile would cover with as much padding as work.
//  * Tile size: relative to a 128 x 256 tile the full tile moves a third
//    fewer bytes from L2 per FLOP, the tall tile 17 % fewer again and reads
//    22 % fewer fragment bytes from LDS per MFMA (a timing variant that ran
//    1.5 times the MFMAs per K step on the same loads took 8 % (up GEMM) and
//    13 % (down GEMM) less time per FLOP on the DeepSeek-V3-shaped shard).
//  * Eight waves: direct-to-LDS loads complete at a rate set by how many
//    waves have loads in flight (about 30 B/clk per CU from four waves, 50
//    from eight, measured on the MI355X), and this tile needs ~32 B/clk per
//    CU at the full MFMA rate.
//  * K advances 32 bf16 (a 64-byte row piece) per step through a four-stage
//    LDS ring of 40 KB stages (room for the wide tile's 640 rows); loads run
//    three steps ahead.  The swizzle for 64-byte rows is
//    chunk ^ ((row >> 2) & 3): the 16 rows read together by one fragment load
//    cover every (row mod 4, chunk) pair, i.e. all LDS banks once.
//  * Work table: one entry per (tile, n-range) unit, built on the device:
//    for each expert, its full tiles for every n-tile (in groups of 8
//    m-tiles, n-tile-major inside a group), then its wide tile for every
//    512-row n-range, cut into 8 contiguous ranges, one per XCD, so an
//    expert's units run together on one XCD and share its operands in L2.
// ---------------------------------------------------------------------------
constexpr int kBigBM = 256, kBigBN = 256;
constexpr int kTallBM = 384;
// Rows per expert (the host's bound, N_cap / E_L) from which the tall tile
// is the full tile.  Measured on arrival-order prefixes of the DeepSeek-V3
// shard: at 1024 rows per expert the tall tile was 7 % slower (more padding
// of 129..383-row remainders), from 1536 on it was faster.
constexpr int kTallMinRows = 1536;
constexpr int kWideBM = 128, kWideBN = 512;
constexpr int kBigThreads = 512;
constexpr int kBigRowBytes = 64;
constexpr int kBigStages = 4;
constexpr int kBigStageBytes = (kWideBM + kWideBN) * kBigRowBytes;  // 40 KB

// Block shapes of the large-tile kernel body: token rows, weight rows, token
// rows per wave (eight waves of WM x 128), LDS stage size and ring depth.
// Full (or tall) and wide tiles share one kernel and so one ring (40 KB
// stages).  (A 128 x 256 shape with four
// waves and 72 KB, two blocks per CU so that one block's first loads and
// epilogue overlap the other's main loop, measured 5-7 % slower.)
template <int BM_, int BN_, int WM_, int STAGE_, int STAGES_>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, kStageBytes = STAGE_, kStages = STAGES_;
  static constexpr int kJ = WM / 32;          // 32-row token blocks per wave
  static constexpr int kWaveRows = BM / WM;   // waves along the token rows
  static constexpr int NW = kWaveRows * (BN / 128);
  static_assert(NW == 8 && WM % 32 == 0 && BM % WM == 0, "eight waves of WM x 128");
  static_assert((BM + BN) * kBigRowBytes <= STAGE_, "a K step fits a stage");
  static_assert(BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "whole 16-row load groups per wave");
};
using FullShape = TileShape<kBigBM, kBigBN, 64, kBigStageBytes, kBigStages>;
using TallShape = TileShape<kTallBM, kBigBN, 96, kBigStageBytes, kBigStages>;
using WideShape = TileShape<kWideBM, kWideBN, 64, kBigStageBytes, kBigStages>;
// The full-tile shape of BM token rows (256: full, 384: tall).
template <int BM> struct FullTile { using type = FullShape; };
template <> struct FullTile<kTallBM> { using type = TallShape; };


// Work units of the large-tile GEMMs (see above).  Entry {expert, first row,
// n-index, wide}: the n-index counts 256-row weight tiles of a full (or tall)
// tile or 512-row ranges of a wide one.  An expert with 129..bm-1 rows past
// its last full tile gets one more full tile instead of a wide one.
__device__ __forceinline__ void expert_units(int cnt, int bm, bool allow_wide, int& full,
                                             int& wide) {
  full = cnt / bm;
  const int rem = cnt - full * bm;
  wide = allow_wide && rem > 0 && rem <= kWideBM;
  if (rem > 0 && !wide) ++full;
}

constexpr int kGroupM = 8;

// Writes one table; the grid's threads take units u = gtid, gtid + threads,
// ... and find the unit's expert by binary search over the experts' first
// units.
__device__ __forceinline__ void write_units(const int* s_start, const int* s_off,
                                            const int* s_full, int E_L, int nt, int total, int bm,
                                            int4* __restrict__ units) {
  const int step = gridDim.x * blockDim.x;
  for (int u = blockIdx.x * blockDim.x + threadIdx.x; u < total; u += step) {
    const int e = run_owner(s_start, E_L, u), v = u - s_start[e], full = s_full[e];
    if (v < full * nt) {
      // groups of kGroupM m-tiles, n-tile-major inside a group, so the 32
      // CUs of an XCD work on about 8 m-tiles x 4 n-tiles of an expert at
      // a time and each operand slab leaves L2 fewer times
      const int g = v / (kGroupM * nt), m0 = g * kGroupM;
      const int gm = min(kGroupM, full - m0), r = v - g * kGroupM * nt;
      units[u] = make_int4(e, s_off[e] + (m0 + r % gm) * bm, r / gm, 0);
    } else
      units[u] = make_int4(e, s_off[e] + full * bm, v - full * nt, 1);
  }
}

__global__ __launch_bounds__(1024) void unit_schedule_kernel(
    const int32_t* __restrict__ seg, int seg_cap, int E_L, int nt_a, int nt_b, int bm, bool allow_wide,
    int4* __restrict__ units_a, int32_t* __restrict__ n_a, int4* __restrict__ units_b,
    int32_t* __restrict__ n_b, int32_t* __restrict__ status, int32_t* __restrict__ tickets) {
  __shared__ int s_off[1024], s_full[1024], s_sa[1024], s_sb[1024];
  const int e = threadIdx.x;
  int cnt = 0, off = 0;
  if (e < E_L) {
    const int2 sg = segment(seg, seg_cap, e);
    off = sg.x;
    cnt = sg.y - sg.x;
  }
  int full, wide;
  expert_units(cnt, bm, allow_wide, full, wide);
  const int nw_a = (nt_a + 1) / 2, nw_b = (nt_b + 1) / 2;
  int tot_a, tot_b;
  const int sa = block_exclusive_scan(full * nt_a + wide * nw_a, &tot_a);
  const int sb = block_exclusive_scan(full * nt_b + wide * nw_b, &tot_b);
  if (e < E_L) {
    s_off[e] = off;
    s_full[e] = full;
    s_sa[e] = sa;
    s_sb[e] = sb;
  }
  __syncthreads();
  write_units(s_sa, s_off, s_full, E_L, nt_a, tot_a, bm, units_a);
  write_units(s_sb, s_off, s_full, E_L, nt_b, tot_b, bm, units_b);
  if (blockIdx.x != 0) return;
  if (e == 0) {
    *n_a = tot_a;
    *n_b = tot_b;
    if (status) *status = 0;
  }
  if (tickets && e < 2 * kXcds) tickets[e] = 0;  // per-XCD unit counters of both GEMMs
}

// Epilogue of a large-tile unit: the wave's WM x 128 accumulators (token
// rows wm*WM.., weight rows wn*128.. of the tile) become bf16 y (staged
// through LDS for whole 256-byte row pieces), GELU h or SwiGLU h.  Every
// wave must be past its last direct load and fragment read of the ring.
template <int MODE, class SH>
__device__ __forceinline__ void big_epilogue(const GemmArgs& g, f32x16 (&acc)[4][SH::kJ], int row0,
                                             int seg_end, int nbase, uint8_t* smem) {
  constexpr int NW = SH::NW, kWaveRows = SH::kWaveRows, WM = SH::WM, kJ = SH::kJ;
  constexpr int kStages = SH::kStages, kStageBytes = SH::kStageBytes;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int wm = w % kWaveRows, wn = w / kWaveRows;
  const int lr = lane & 31;
  const int cq = (lane >> 5) * 4;
  uint16_t* C = static_cast<uint16_t*>(g.C);
  if constexpr (MODE == MODE_PLAIN) {
    // The wave's WM x 128 result goes through LDS, 64 rows at a time, so
    // that the stores write whole 256-byte row pieces (16 lanes per row, 4
    // rows per instruction) instead of 16 bytes of 32 rows each.  Every wave
    // is past its last fragment read and direct load once all have reached
    // the barrier; then each wave uses its own 64-row region (its reads of a
    // piece are done before it writes the next: LDS runs a wave's accesses
    // in order).
    constexpr int kPitch = 272;  // 256 bytes + 16: rows start 4 banks apart
    static_assert(NW * 64 * kPitch <= kStages * kStageBytes, "epilogue tile fits the ring");
    __builtin_amdgcn_s_barrier();
    uint8_t* stile = smem + w * 64 * kPitch;
    const int col = nbase + wn * 128 + (lane & 15) * 8;
#pragma unroll
    for (int j0 = 0; j0 < kJ; j0 += 2) {
      constexpr int kPiece = 2;  // token blocks per piece (the last may hold one)
      const int jn = kJ - j0 < kPiece ? kJ - j0 : kPiece;
#pragma unroll
      for (int jj = 0; jj < kPiece; ++jj) {
        if (jj >= jn) break;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint2 o;
            o.x = pack_bf16x2(acc[i][j0 + jj][q * 4 + 0], acc[i][j0 + jj][q * 4 + 1]);
            o.y = pack_bf16x2(acc[i][j0 + jj][q * 4 + 2], acc[i][j0 + jj][q * 4 + 3]);
            *reinterpret_cast<uint2*>(stile + (jj * 32 + lr) * kPitch + (i * 32 + q * 8 + cq) * 2) = o;
          }
      }
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        if (it >= jn * 8) break;
        const int rl = it * 4 + (lane >> 4);
        const uint4 v = *reinterpret_cast<const uint4*>(stile + rl * kPitch + (lane & 15) * 16);
        const int m = row0 + wm * WM + j0 * 32 + rl;
        if (m < seg_end && col < g.Nout)
          *reinterpret_cast<uint4*>(C + static_cast<int64_t>(m) * g.Nout + col) = v;
      }
    }
  } else if constexpr (MODE == MODE_GELU) {
    // h = gelu(x W1^T), panel or row major
    uint8_t* C8 = reinterpret_cast<uint8_t*>(C);
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int m = row0 + wm * WM + j * 32 + lr;
      if (m >= seg_end) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nbase + wn * 128 + i * 32 + q * 8 + cq;
          if (col >= g.Nout) continue;
          uint2 o;
          o.x = pack_bf16x2(gelu_f(acc[i][j][q * 4 + 0]), gelu_f(acc[i][j][q * 4 + 1]));
          o.y = pack_bf16x2(gelu_f(acc[i][j][q * 4 + 2]), gelu_f(acc[i][j][q * 4 + 3]));
          *reinterpret_cast<uint2*>(C8 + out_offset(g, m, col)) = o;
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int m = row0 + wm * WM + j * 32 + lr;
      if (m >= seg_end) continue;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nbase + wn * 64 + hb * 32 + q * 8 + cq;
          if (col >= g.Nout) continue;
          float hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gt = acc[hb][j][q * 4 + r], up = acc[hb + 2][j][q * 4 + r];
            hv[r] = silu_mul(gt, up);
          }
          uint2 o;
          o.x = pack_bf16x2(hv[0], hv[1]);
          o.y = pack_bf16x2(hv[2], hv[3]);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(C) + out_offset(g, m, col)) = o;
        }
    }
  }
}


template <int MODE, class SH>
__device__ __forceinline__ void big_tile(const GemmArgs& g, const int4 unit, uint8_t* smem) {
  constexpr bool kSwiglu = MODE == MODE_SWIGLU || MODE == MODE_SWIGLU_FP8OUT;
  constexpr int BM = SH::BM, BN = SH::BN, NW = SH::NW;
  constexpr int kStages = SH::kStages, kStageBytes = SH::kStageBytes, kAhead = kStages - 1;
  constexpr int kWRegion = BM * kBigRowBytes;
  constexpr int kAGroups = BM / 16;                        // 16-row load groups
  constexpr int kLoads = (BM + BN) / 16 / NW;              // per wave and step: 4 or 5
  constexpr int kALoads = kAGroups / NW;                   // of which A: 2, 3 or 1
  constexpr int kWaveRows = SH::kWaveRows, WM = SH::WM, kJ = SH::kJ;
  constexpr int kFrag = 4 + kJ;                            // fragment reads per K half

  const int e = unit.x, row0 = unit.y, nidx = unit.z;
  const int seg_end = segment(g.seg, g.seg_cap, e).y;
  const int ldb = 2 * g.K;
  const int nk = ldb / kBigRowBytes;
  // Buffer views advance one 64-byte K piece per step (see the pipelined
  // kernel); rows past the segment read zeros.
  const int64_t a_skip = g.a_index ? 0 : static_cast<int64_t>(row0) * g.a_rs;
  const uint8_t* a_base = g.A + a_skip;
  const int64_t a_left = g.a_bytes - a_skip;
  const uint8_t* w_base = g.W + e * g.w_stride;
  // first output column (SwiGLU: of h) and first weight row of the unit
  const int nbase = kSwiglu ? nidx * (BN / 2) : nidx * BN;

  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  // direct loads: wave w moves A groups w*kALoads.. and W groups
  // kAGroups + w*(kLoads - kALoads)..; A rows come first in the stage.
  int voff[kLoads], ldst[kLoads];
#pragma unroll
  for (int q = 0; q < kLoads; ++q) {
    const int grp = q < kALoads ? w * kALoads + q : kAGroups + w * (kLoads - kALoads) + (q - kALoads);
    const int rr = grp * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ ((rr >> 2) & 3);
    if (rr < BM) {
      const bool valid = row0 + rr < seg_end;
      const int arow = g.a_index && valid ? g.a_index[row0 + rr] : rr;
      voff[q] = valid ? arow * g.a_rs + chunk * 16 : kOobOffset;
    } else {
      const int r = rr - BM;
      int grow;
      if (kSwiglu)
        grow = r < BN / 2 ? min(nbase + r, g.Nout - 1)
                          : g.Nout + min(nbase + (r - BN / 2), g.Nout - 1);
      else
        grow = min(nbase + r, g.NW - 1);
      voff[q] = grow * g.w_rs + chunk * 16;
    }
    ldst[q] = grp * 1024;
  }
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(a_base, a_left);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(w_base, g.w_stride);
  auto dma = [&](int step, int stage) {
    // steps past the last one load nothing (out-of-range offsets), which
    // keeps the per-step load count that the waits rely on
    const bool live = step < nk;
    const int k = live ? step : 0;
    uint8_t* base = smem + stage * kStageBytes;
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(q < kALoads ? rA : rW, (lds_ptr_t)(base + ldst[q]),
                                               16, live ? voff[q] : kOobOffset,
                                               k * (q < kALoads ? g.a_cs : g.w_cs), 0, 0);
  };

  const int wm = w % kWaveRows, wn = w / kWaveRows;
  const int lr = lane & 31, hi = lane >> 5, sl = (lr >> 2) & 3;
  int foff[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) foff[kk] = lr * kBigRowBytes + (((2 * kk) | hi) ^ sl) * 16;
  // LDS row (in the weight region) of the wave's weight block i
  int wbase[4], abase[kJ];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = kSwiglu ? (i < 2 ? 0 : BN / 2) + wn * 64 + (i & 1) * 32 : wn * 128 + i * 32;
    wbase[i] = kWRegion + row * kBigRowBytes;
  }
#pragma unroll
  for (int j = 0; j < kJ; ++j) abase[j] = (wm * WM + j * 32) * kBigRowBytes;

  f32x16 acc[4][kJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  bf16x8 fa[2][4], fb[2][kJ];
  auto lfrag = [&](const uint8_t* st, int kk, int set) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[set][i] = *reinterpret_cast<const bf16x8*>(st + wbase[i] + foff[kk]);
#pragma unroll
    for (int j = 0; j < kJ; ++j) fb[set][j] = *reinterpret_cast<const bf16x8*>(st + abase[j] + foff[kk]);
  };
  auto mma = [&](int set, int first, int count) {
#pragma unroll
    for (int q = first; q < first + count; ++q) {
      const int i = q / kJ, j = q % kJ;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
    }
  };

#pragma unroll
  for (int st = 0; st < kAhead; ++st) dma(st, st);
  WAIT_VMCNT((kAhead - 1) * kLoads);
  __builtin_amdgcn_s_barrier();
  if constexpr (kJ > 2) {
    // 96-row waves: the 192 sums leave room for one set of fragments, so
    // each K half reads its fragments and then runs its MFMAs (the other
    // wave of the SIMD covers the read latency).
    int s_cur = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const uint8_t* cur = smem + s_cur * kStageBytes;
      dma(kt + kAhead, s_cur == 0 ? kStages - 1 : s_cur - 1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        lfrag(cur, kk, 0);
        mma(0, 0, 4 * kJ);
      }
      WAIT_VMCNT_LDS((kAhead - 1) * kLoads);
      __builtin_amdgcn_s_barrier();
      s_cur = s_cur + 1 == kStages ? 0 : s_cur + 1;
    }
    WAIT_VMCNT(0);
    big_epilogue<MODE, SH>(g, acc, row0, seg_end, nbase, smem);
    return;
  }
  lfrag(smem, 0, 0);

  int s_cur = 0;  // stage of step kt
  for (int kt = 0; kt < nk; ++kt) {
    const int s_nxt = s_cur + 1 == kStages ? 0 : s_cur + 1;
    const uint8_t* cur = smem + s_cur * kStageBytes;
    const uint8_t* nxt = smem + s_nxt * kStageBytes;
    // The stage of step kt - 1 was released by the barrier that ended that
    // step; it takes step kt + kAhead.
    dma(kt + kAhead, s_cur == 0 ? kStages - 1 : s_cur - 1);
    lfrag(cur, 1, 1);
    mma(0, 0, 4 * kJ);
    // the second K half's fragment reads and the step's loads go between
    // the first half's MFMAs
#pragma unroll
    for (int q = 0; q < kFrag; ++q) {
      SCHED(kSchedMfma, 1);
      SCHED(kSchedDsRead, 1);
      if (q < kLoads) SCHED(kSchedVmemRead, 1);
    }
    SCHED(kSchedMfma, 4 * kJ - kFrag);
    mma(1, 0, 2 * kJ);
    // Step boundary: step kt+1 has landed once only the later steps are in
    // flight; this wave's reads of stage kt are done.
    WAIT_VMCNT_LDS((kAhead - 1) * kLoads);
    __builtin_amdgcn_s_barrier();
    lfrag(nxt, 0, 0);
    mma(1, 2 * kJ, 2 * kJ);
#pragma unroll
    for (int q = 0; q < 2 * kJ; ++q) {
      SCHED(kSchedDsRead, 2);
      SCHED(kSchedMfma, 1);
    }
    s_cur = s_nxt;
  }
  WAIT_VMCNT(0);
  big_epilogue<MODE, SH>(g, acc, row0, seg_end, nbase, smem);
}

// ---------------------------------------------------------------------------
// Persistent large-tile GEMM with the SwiGLU or GELU epilogue (the up GEMM,
// whose epilogue stores h straight from the accumulators and leaves the LDS
// alone).  One block per CU pulls units from its XCD's queue -- the XCD's
// contiguous range of the unit table, handed out by an atomic counter -- so
// that CUs that finish early take more units (the tile-granular work of page
// "ExpertPlex"'s persistent kernels; the tail effect of page "CascadeEP
// ...", section 3.2, is the last round of units).  Between two full units
// the load ring runs on: the last three K steps of a unit load the first
// three steps of the next one, whose ticket the block took when it began the
// unit, so those loads are in flight while the unit's epilogue runs and the
// next unit starts without an empty pipeline.  A wide unit (a segment's
// remainder, different tile shape) never chains: before it the ring drains
// and it runs as in the one-unit-per-block kernel.  (The down GEMM's
// epilogue stages its tile through the whole ring, so it keeps one block
// per unit; chaining it through the one free ring stage, 16 token rows per
// wave at a time, measured 3-5 % slower.)
// ---------------------------------------------------------------------------
// The wide unit of both large-tile kernels (one call site of the big_tile
// specialisation: the host pass of hipcc rejects a second one).
template <int MODE>
__device__ __forceinline__ void big_tile_wide(const GemmArgs& g, const int4 unit, uint8_t* smem) {
  big_tile<MODE, WideShape>(g, unit, smem);
}

template <int MODE, int BM_>
struct BigChain {
  using SH = typename FullTile<BM_>::type;
  static constexpr bool kSwiglu = MODE == MODE_SWIGLU;
  static constexpr int BM = SH::BM, BN = SH::BN, NW = SH::NW;
  static constexpr int kStages = SH::kStages, kStageBytes = SH::kStageBytes;
  static constexpr int kAhead = kStages - 1;
  static constexpr int kWRegion = BM * kBigRowBytes;
  static constexpr int kAGroups = BM / 16;
  static constexpr int kLoads = (BM + BN) / 16 / NW;   // 4 (full) or 5 (tall)
  static constexpr int kALoads = kAGroups / NW;        // 2 or 3

  // Load addressing of one unit (lane offsets, buffer views) and its place.
  struct Unit {
    int row0, seg_end, nbase;
    int voff[kLoads];
    __amdgpu_buffer_rsrc_t rA, rW;
  };

  __device__ static Unit setup(const GemmArgs& g, const int4 unit) {
    Unit u;
    const int e = unit.x;
    u.row0 = unit.y;
    u.seg_end = segment(g.seg, g.seg_cap, e).y;
    u.nbase = kSwiglu ? unit.z * (BN / 2) : unit.z * BN;
    const int64_t a_skip = g.a_index ? 0 : static_cast<int64_t>(u.row0) * g.a_rs;
    const int lane = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int grp = q < kALoads ? w * kALoads + q : kAGroups + w * (kLoads - kALoads) + (q - kALoads);
      const int rr = grp * 16 + (lane >> 2);
      const int chunk = (lane & 3) ^ ((rr >> 2) & 3);
      if (rr < BM) {
        const bool valid = u.row0 + rr < u.seg_end;
        const int arow = g.a_index && valid ? g.a_index[u.row0 + rr] : rr;
        u.voff[q] = valid ? arow * g.a_rs + chunk * 16 : kOobOffset;
      } else {
        const int r = rr - BM;
        int grow;
        if (kSwiglu)
          grow = r < BN / 2 ? min(u.nbase + r, g.Nout - 1)
                            : g.Nout + min(u.nbase + (r - BN / 2), g.Nout - 1);
        else
          grow = min(u.nbase + r, g.NW - 1);
        u.voff[q] = grow * g.w_rs + chunk * 16;
      }
    }
    u.rA = make_rsrc(g.A + a_skip, g.a_bytes - a_skip);
    u.rW = make_rsrc(g.W + e * g.w_stride, g.w_stride);
    return u;
  }

  // The loads of K step `step` of unit u into `stage` (live == false: the
  // same number of loads, out of range, so the wait counts hold).
  __device__ static void dma(const GemmArgs& g, const Unit& u, bool live, int step, int stage,
                             uint8_t* smem) {
    const int lane_grp = threadIdx.x >> 6;
    uint8_t* base = smem + stage * kStageBytes;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int grp = q < kALoads ? lane_grp * kALoads + q
                                  : kAGroups + lane_grp * (kLoads - kALoads) + (q - kALoads);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(q < kALoads ? u.rA : u.rW,
                                               (lds_ptr_t)(base + grp * 1024), 16,
                                               live ? u.voff[q] : kOobOffset,
                                               live ? step * (q < kALoads ? g.a_cs : g.w_cs) : 0,
                                               0, 0);
    }
  }
};

template <int MODE, int BM>
__global__ __launch_bounds__(kBigThreads, 1) void gemm_big_persistent_kernel(const GemmArgs g) {
  using C = BigChain<MODE, BM>;
  using SH = typename C::SH;
  constexpr int kStages = C::kStages, kStageBytes = C::kStageBytes, kAhead = C::kAhead;
  constexpr int kLoads = C::kLoads;
  constexpr bool kSwiglu = C::kSwiglu;
  constexpr int WM = SH::WM, kJ = SH::kJ, kFrag = 4 + kJ;
  static_assert(kJ == 2, "the chained kernel runs 64-row waves (two fragment sets)");
  // The ring takes the whole LDS (no static __shared__ variable fits beside
  // it): the ticket is passed through a word of a stage that holds nothing
  // in flight or still to be read (slot, a byte offset).
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int total = *g.n_tiles;
  const int per_xcd = ceil_div(total, kXcds);
  const int x = blockIdx.x % kXcds;  // blocks go to the XCDs round-robin by id
  const int q0 = x * per_xcd, q1 = min(total, q0 + per_xcd);
  int32_t* ctr = g.tickets + x;
  // the next unit of this XCD's queue (-1: none left); every thread calls it
  auto take = [&](int slot) -> int {
    int* tk = reinterpret_cast<int*>(smem + slot);
    __syncthreads();  // every earlier LDS read of the block is done
    if (threadIdx.x == 0) *tk = atomicAdd(ctr, 1);
    __syncthreads();
    const int t = q0 + *tk;
    __syncthreads();  // every thread has the ticket before the slot is reused
    return t < q1 ? t : -1;
  };
  const int nk = 2 * g.K / kBigRowBytes;

  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int wm = w % SH::kWaveRows, wn = w / SH::kWaveRows;
  const int lr = lane & 31, hi = lane >> 5, sl = (lr >> 2) & 3;
  int foff[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) foff[kk] = lr * kBigRowBytes + (((2 * kk) | hi) ^ sl) * 16;
  int wbase[4], abase[kJ];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = kSwiglu ? (i < 2 ? 0 : SH::BN / 2) + wn * 64 + (i & 1) * 32 : wn * 128 + i * 32;
    wbase[i] = C::kWRegion + row * kBigRowBytes;
  }
#pragma unroll
  for (int j = 0; j < kJ; ++j) abase[j] = (wm * WM + j * 32) * kBigRowBytes;

  f32x16 acc[4][kJ];
  bf16x8 fa[2][4], fb[2][kJ];
  auto lfrag = [&](const uint8_t* st, int kk, int set) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[set][i] = *reinterpret_cast<const bf16x8*>(st + wbase[i] + foff[kk]);
#pragma unroll
    for (int j = 0; j < kJ; ++j) fb[set][j] = *reinterpret_cast<const bf16x8*>(st + abase[j] + foff[kk]);
  };
  auto mma = [&](int set, int first, int count) {
#pragma unroll
    for (int q = first; q < first + count; ++q) {
      const int i = q / kJ, j = q % kJ;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
    }
  };
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  };

  int t = take(0);  // nothing in flight yet
  while (t >= 0) {
    int4 unit = g.info[t];
    if (unit.w) {  // a wide unit: its own prologue, loop and epilogue
      big_tile_wide<MODE>(g, unit, smem);
      t = take(0);  // its loads have all landed and its epilogue uses no LDS
      continue;
    }
    // A chain of full units.  Prologue of the first one.
    typename C::Unit cur = C::setup(g, unit);
#pragma unroll
    for (int st = 0; st < kAhead; ++st) C::dma(g, cur, true, st, st, smem);
    WAIT_VMCNT((kAhead - 1) * kLoads);
    __builtin_amdgcn_s_barrier();
    lfrag(smem, 0, 0);
    int s_cur = 0;  // ring stage of the current step
    for (;;) {
      zero_acc();
      // the next unit: chained if it is a full one.  The stage before the
      // current step's (the previous unit's last step, or the one the
      // prologue left empty) is free until this unit's step 3 is loaded.
      const int tn = take((s_cur == 0 ? kStages - 1 : s_cur - 1) * kStageBytes);
      const int4 un = tn >= 0 ? g.info[tn] : make_int4(0, 0, 0, 1);
      const bool chain = tn >= 0 && !un.w;
      typename C::Unit nxt = chain ? C::setup(g, un) : cur;
      for (int kt = 0; kt < nk; ++kt) {
        const int s_nxt = s_cur + 1 == kStages ? 0 : s_cur + 1;
        const uint8_t* st_cur = smem + s_cur * kStageBytes;
        const uint8_t* st_nxt = smem + s_nxt * kStageBytes;
        // step kt + kAhead of the stream: this unit's, else the next unit's
        // first steps (or out-of-range loads at the end of a chain)
        const int ls = kt + kAhead;
        const int lstage = s_cur == 0 ? kStages - 1 : s_cur - 1;
        if (ls < nk)
          C::dma(g, cur, true, ls, lstage, smem);
        else
          C::dma(g, nxt, chain, ls - nk, lstage, smem);
        lfrag(st_cur, 1, 1);
        mma(0, 0, 4 * kJ);
#pragma unroll
        for (int q = 0; q < kFrag; ++q) {
          SCHED(kSchedMfma, 1);
          SCHED(kSchedDsRead, 1);
          if (q < kLoads) SCHED(kSchedVmemRead, 1);
        }
        SCHED(kSchedMfma, 4 * kJ - kFrag);
        mma(1, 0, 2 * kJ);
        WAIT_VMCNT_LDS((kAhead - 1) * kLoads);
        __builtin_amdgcn_s_barrier();
        lfrag(st_nxt, 0, 0);
        mma(1, 2 * kJ, 2 * kJ);
#pragma unroll
        for (int q = 0; q < 2 * kJ; ++q) {
          SCHED(kSchedDsRead, 2);
          SCHED(kSchedMfma, 1);
        }
        s_cur = s_nxt;
      }
      if (!chain) WAIT_VMCNT(0);  // the out-of-range loads of the chain's end
      // SwiGLU / GELU epilogue: stores from the accumulators, no LDS
      big_epilogue<MODE, SH>(g, acc, cur.row0, cur.seg_end, cur.nbase, smem);
      if (!chain) {
        t = tn;
        break;
      }
      cur = nxt;
    }
  }
}

template <int MODE, int BM>
__global__ __launch_bounds__(kBigThreads, 1) void gemm_big_kernel(const GemmArgs g) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int total = *g.n_tiles;
  const int per_xcd = ceil_div(total, kXcds);
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int t = (blockIdx.x % kXcds) * per_xcd + slot;
  if (t >= total) return;
  const int4 unit = g.info[t];
  if (unit.w)
    big_tile_wide<MODE>(g, unit, smem);
  else
    big_tile<MODE, typename FullTile<BM>::type>(g, unit, smem);
}


// Compute units of the current device (looked up once per device).
inline int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cus[dev].load(std::memory_order_acquire);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  cus[dev].store(n, std::memory_order_release);
  return n;
}

template <int MODE, int BM>
hipError_t launch_big(const GemmArgs& g, int64_t max_units, hipStream_t s) {
  static_assert(kBigStages * kBigStageBytes <= 160 * 1024, "the ring fits the CU's LDS");
  const size_t lds = kBigStages * kBigStageBytes;
  auto kern = gemm_big_kernel<MODE, BM>;
  // Persistent for the 256-row tile only: with 96-row waves the two units'
  // load state the chain holds does not fit beside the 192 sums (it spilled
  // to scratch and ran 9 % slower than one block per unit).
  if constexpr ((MODE == MODE_SWIGLU || MODE == MODE_GELU) && BM == kBigBM) {
    if (g.tickets) {  // persistent: one block per CU (at most one unit each, at least 8)
      auto pkern = gemm_big_persistent_kernel<MODE, BM>;
      static std::atomic<uint64_t> lds_set_p{0};
      allow_dynamic_lds(reinterpret_cast<const void*>(pkern), static_cast<int>(lds), lds_set_p);
      int64_t blocks = device_cus();
      blocks = blocks < max_units ? blocks : max_units;
      blocks = (blocks + kXcds - 1) / kXcds * kXcds;
      hipLaunchKernelGGL(pkern, dim3(static_cast<unsigned>(blocks)), dim3(kBigThreads), lds, s, g);
      return hipGetLastError();
    }
  }
  static std::atomic<uint64_t> lds_set{0};
  allow_dynamic_lds(reinterpret_cast<const void*>(kern), static_cast<int>(lds), lds_set);
  const int64_t blocks = (max_units + kXcds - 1) / kXcds * kXcds + kXcds;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kBigThreads), lds, s, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Large-tile block-FP8 kernel: 8 waves (two per SIMD) as 4 (token rows) x 2
// (weight rows) over a 256 x 256 tile, each wave 64 x 128 (2 x 4 MFMA 32x32
// tiles).  One K step is one 128-wide scale block: 128 bytes of every row
// through an LDS ring (codes plus the step's token scales, all by direct
// loads).
//  * Scales: for each 32x32 tile the two MFMAs of the step (K 0..63, 64..127)
//    run into a fresh accumulator (the MFMA's zero input) that is then added
//    to the tile's sum times (weight block scale x token group scale).  At
//    64 x 128 per wave the sums (128 registers per lane) stay in VGPRs, so a
//    tile's promotion is 16 FMAs; the two waves of a SIMD overlap one's
//    promotion with the other's MFMAs.  (With 128 x 128 per wave the 256 sums
//    could not all be VGPRs and every promotion moved them through AGPRs:
//    about 60 VALU instructions per tile and step, more issue time than the
//    step's MFMAs.)
//  * Fused gather: with a_index, token row j is row a_index[j] of the codes
//    and of the scales.
// ---------------------------------------------------------------------------
constexpr int kF8BN = 256;
constexpr int kF8RowBytes = 128;
constexpr int kF8Pitch = 272;  // bf16 epilogue rows
constexpr int kCuLds = 160 * 1024;  // LDS of a CU: static plus dynamic must fit

template <int WM, int WAVES_M>
struct F8Tile {
  static constexpr int BM = WAVES_M * WM;
  static constexpr int kWaves = 2 * WAVES_M;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kScaleOff = (BM + kF8BN) * kF8RowBytes;
  static constexpr int kStageBytes = kScaleOff + BM * 4 + 512;
  static constexpr int kStatic = 2 * BM * 4;         // row_amax
  static constexpr int kRoom = kCuLds - kStatic;
  static constexpr int kStages = kRoom / kStageBytes < 3 ? kRoom / kStageBytes : 3;
  static constexpr int kEpilogue = kWaves * WM * kF8Pitch;
  // dynamic LDS: the ring, or the bf16 epilogue tile if larger
  static constexpr int kLds =
      kStages * kStageBytes > kEpilogue ? kStages * kStageBytes : kEpilogue;
  static constexpr int kALoads = BM / 8 / kWaves;     // 8-row groups of A per wave
  static constexpr int kWLoads = kF8BN / 8 / kWaves;  // 8-row groups of W per wave
  static constexpr int kLoads = kALoads + kWLoads;
  static constexpr int kJ = WM / 32;                  // token blocks per wave
  static_assert(kStages >= 2, "LDS ring");
  static_assert(kLds + kStatic <= kCuLds, "static plus dynamic LDS fit the CU");
  static_assert(BM % (8 * kWaves) == 0 && kF8BN % (8 * kWaves) == 0, "whole load groups");
  static_assert(BM % 64 == 0, "token scales in 64-row pieces");
};

template <int MODE, int WM, int WAVES_M>
__device__ __forceinline__ void big_fp8_tile(const GemmArgs& g) {
  using TT = F8Tile<WM, WAVES_M>;
  constexpr int BM = TT::BM;
  constexpr int kStages = TT::kStages, kAhead = kStages - 1;
  constexpr int kLoads = TT::kLoads, kALoads = TT::kALoads, kWLoads = TT::kWLoads;
  constexpr int kJ = TT::kJ;
  constexpr int kDma = kLoads + 1;  // + the token-scale load
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  __shared__ float row_amax[2][BM];
  constexpr bool kSwiglu = MODE == MODE_SWIGLU || MODE == MODE_SWIGLU_FP8OUT;

  const int total = *g.n_tiles;
  const int per_xcd = ceil_div(total, kXcds);
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int t = (blockIdx.x % kXcds) * per_xcd + slot;
  if (t >= total) return;
  const int4 unit = g.info[t];
  const int e = unit.x, row0 = unit.y, nt = unit.z;
  const int seg_end = segment(g.seg, g.seg_cap, e).y;
  const int ldb = g.K;               // bytes per row of A and W
  const int nk = g.K / 128;
  const int kb_n = g.K / 128;        // scale blocks per row

  const int64_t a_skip = g.a_index ? 0 : static_cast<int64_t>(row0) * ldb;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + a_skip, g.a_bytes - a_skip);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.W + e * g.w_stride, g.w_stride);
  const __amdgpu_buffer_rsrc_t rS =
      make_rsrc(g.A_scale + (g.a_index ? 0 : static_cast<int64_t>(row0) * kb_n),
                (g.a_bytes / ldb - (g.a_index ? 0 : row0)) * kb_n * 4);
  const int nbase = kSwiglu ? nt * (kF8BN / 2) : nt * kF8BN;

  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  // direct loads: wave w moves A groups w*kALoads.. and W groups
  // BM/8 + w*kWLoads .. (8 rows of 128 bytes each), and the token scales of
  // 64 rows ((w % (BM/64)) * 64 ..; waves w and w + BM/64 load the same rows).
  int voff[kLoads], ldst[kLoads];
#pragma unroll
  for (int q = 0; q < kLoads; ++q) {
    const int grp = q < kALoads ? w * kALoads + q : BM / 8 + w * kWLoads + (q - kALoads);
    const int rr = grp * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((rr >> 1) & 7);
    if (rr < BM) {
      const bool valid = row0 + rr < seg_end;
      const int arow = g.a_index && valid ? g.a_index[row0 + rr] : rr;
      voff[q] = valid ? arow * ldb + chunk * 16 : kOobOffset;
    } else {
      const int r = rr - BM;
      int grow;
      if (kSwiglu)
        grow = r < kF8BN / 2 ? min(nbase + r, g.Nout - 1)
                             : g.Nout + min(nbase + (r - kF8BN / 2), g.Nout - 1);
      else
        grow = min(nbase + r, g.NW - 1);
      voff[q] = grow * ldb + chunk * 16;
    }
    ldst[q] = grp * 1024;
  }
  const int srow = (w % (BM / 64)) * 64;
  int soff;
  {
    const int rr = srow + lane;
    const bool valid = row0 + rr < seg_end;
    const int arow = g.a_index && valid ? g.a_index[row0 + rr] : rr;
    soff = valid ? arow * kb_n * 4 : kOobOffset;
  }
  auto dma = [&](int step, int stage) {
    const int k = min(step, nk - 1);
    uint8_t* base = smem + stage * TT::kStageBytes;
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(q < kALoads ? rA : rW, (lds_ptr_t)(base + ldst[q]),
                                               16, voff[q], k * 128, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_ptr_t)(base + TT::kScaleOff + srow * 4), 4,
                                             soff, k * 4, 0, 0);
  };

  // ---- fragments: lane reads 32 bytes (K 32 hi .. 32 hi + 31 of the
  // sub-step's 64) of row lr of a 32-row block, as two swizzled 16-byte chunks
  const int wm = w % WAVES_M, wn = w / WAVES_M;
  const int lr = lane & 31, hi = lane >> 5, sl = (lr >> 1) & 7;
  int foff[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int c0 = (4 * kk + 2 * hi) ^ sl;
    foff[kk][0] = lr * kF8RowBytes + c0 * 16;
    foff[kk][1] = lr * kF8RowBytes + (c0 ^ 1) * 16;
  }
  int wbase[4], abase[kJ];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = kSwiglu ? (i < 2 ? 0 : kF8BN / 2) + wn * 64 + (i & 1) * 32 : wn * 128 + i * 32;
    wbase[i] = BM * kF8RowBytes + row * kF8RowBytes;
  }
#pragma unroll
  for (int j = 0; j < kJ; ++j) abase[j] = (wm * WM + j * 32) * kF8RowBytes;
  // weight block scales: uniform per wave, scalar loads
  const float* wsc = g.W_scale + e * g.ws_stride;
  const float* swp[2];
  if (kSwiglu) {
    swp[0] = wsc + static_cast<int64_t>(min(nbase, g.Nout - 1) / 128) * kb_n;
    swp[1] = wsc + static_cast<int64_t>((g.Nout + min(nbase, g.Nout - 1)) / 128) * kb_n;
  } else {
    swp[0] = swp[1] =
        wsc + static_cast<int64_t>(min(nbase + __builtin_amdgcn_readfirstlane(wn) * 128,
                                       g.NW - 1) / 128) * kb_n;
  }
  auto wscale = [&](int which, int k) {
    return ((const __attribute__((address_space(4))) float*)(uintptr_t)swp[which])[k];
  };

  f32x16 acc[4][kJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto rd32 = [&](const uint8_t* p0, const uint8_t* p1) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(p0), h4 = *reinterpret_cast<const i32x4*>(p1);
    return i32x8{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
  };

#pragma unroll
  for (int st = 0; st < kAhead; ++st) dma(st, st);
  WAIT_VMCNT((kAhead - 1) * kDma);
  __builtin_amdgcn_s_barrier();

  int s_cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const uint8_t* st = smem + s_cur * TT::kStageBytes;
    // the stage before this one was released by the barrier that ended
    // step kt - 1; it takes step kt + kAhead
    dma(kt + kAhead, s_cur == 0 ? kStages - 1 : s_cur - 1);
    const float sw0 = wscale(0, kt), sw1 = wscale(1, kt);
    // token fragments for the whole step; weight fragments one 32-row block
    // at a time (fewer live registers: the sums take 128)
    i32x8 fb[2][kJ];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < kJ; ++j)
        fb[kk][j] = rd32(st + abase[j] + foff[kk][0], st + abase[j] + foff[kk][1]);
    float sx[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      sx[j] = *reinterpret_cast<const float*>(st + TT::kScaleOff + (wm * WM + j * 32 + lr) * 4);
    const f32x16 zero = {0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const i32x8 fa0 = rd32(st + wbase[i] + foff[0][0], st + wbase[i] + foff[0][1]);
      const i32x8 fa1 = rd32(st + wbase[i] + foff[1][0], st + wbase[i] + foff[1][1]);
      // both token blocks' MFMAs before either promotion: one tile's
      // result latency hides behind the other's MFMAs
      f32x16 tt[kJ];
#pragma unroll
      for (int j = 0; j < kJ; ++j)
        tt[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa0, fb[0][j], zero, 0, 0, 0, 0,
                                                               0, 0);
#pragma unroll
      for (int j = 0; j < kJ; ++j)
        tt[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa1, fb[1][j], tt[j], 0, 0, 0, 0,
                                                               0, 0);
      const float swi = kSwiglu && i >= 2 ? sw1 : sw0;
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const float c = swi * sx[j];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] += tt[j][r] * c;
      }
    }
    // Step boundary: step kt+1 has landed once only the later steps' loads
    // are in flight, and this wave's reads of stage kt are done; the barrier
    // publishes both.
    WAIT_VMCNT_LDS((kAhead - 1) * kDma);
    __builtin_amdgcn_s_barrier();
    s_cur = s_cur + 1 == kStages ? 0 : s_cur + 1;
  }
  WAIT_VMCNT(0);
  __builtin_amdgcn_s_barrier();

  const int cq = (lane >> 5) * 4;
  if constexpr (MODE == MODE_PLAIN) {
    // bf16 rows through LDS: 256-byte row pieces per 16 lanes (see the
    // bf16 large-tile kernel); the barrier above freed the ring.
    uint16_t* C = static_cast<uint16_t*>(g.C);
    uint8_t* stile = smem + w * WM * kF8Pitch;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 o;
          o.x = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
          o.y = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
          *reinterpret_cast<uint2*>(stile + (j * 32 + lr) * kF8Pitch + (i * 32 + q * 8 + cq) * 2) = o;
        }
    const int col = nbase + wn * 128 + (lane & 15) * 8;
#pragma unroll 4
    for (int it = 0; it < WM / 4; ++it) {
      const int rl = it * 4 + (lane >> 4);
      const uint4 v = *reinterpret_cast<const uint4*>(stile + rl * kF8Pitch + (lane & 15) * 16);
      const int m = row0 + wm * WM + rl;
      if (m < seg_end && col < g.Nout)
        *reinterpret_cast<uint4*>(C + static_cast<int64_t>(m) * g.Nout + col) = v;
    }
  } else {
    static_assert(MODE == MODE_SWIGLU_FP8OUT, "block-FP8 h output only");
    // h = silu(gate) * up; the block's 128 h columns are one quantisation
    // group, split over the two waves of a row range (64 columns each)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[hb][j][r] = silu_mul(acc[hb][j][r], acc[hb + 2][j][r]);
    float amax[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      float m = 0.0f;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[hb][j][r]));
      m = fmaxf(m, __shfl_xor(m, 32));
      amax[j] = m;
      if (lane < 32) row_amax[wn][wm * WM + j * 32 + lr] = m;
    }
    __syncthreads();
    uint8_t* C = static_cast<uint8_t*>(g.C);
    const int groups = g.Nout / 128;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int lrow = wm * WM + j * 32 + lr;
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
          *reinterpret_cast<uint32_t*>(crow + nbase + wn * 64 + hb * 32 + q * 8 + cq) = v;
        }
      if (wn == 0 && lane < 32) g.C_scale[static_cast<int64_t>(m) * groups + nt] = sc;
    }
  }
}

// Geometry of the block-FP8 large-tile kernel: 64 rows per wave, 4 waves
// along the rows, so a 256 x 256 tile.  (4 waves of 128 x 128 on the same
// tile spent more VALU issue on the scale promotion than MFMA time.)
constexpr int kF8WM = 64, kF8WavesM = 4;
using F8Big = F8Tile<kF8WM, kF8WavesM>;
constexpr int kF8BM = F8Big::BM;
constexpr int kF8Threads = F8Big::kThreads;

// (A kernel template over MODE only: the tile body takes the geometry.)
template <int MODE>
__global__ __launch_bounds__(kF8Threads, 1) void gemm_big_fp8_kernel(const GemmArgs g) {
  big_fp8_tile<MODE, kF8WM, kF8WavesM>(g);
}

template <int MODE>
hipError_t launch_big_fp8(const GemmArgs& g, int64_t max_units, hipStream_t s) {
  auto kern = gemm_big_fp8_kernel<MODE>;
  static std::atomic<uint64_t> lds_set{0};
  allow_dynamic_lds(reinterpret_cast<const void*>(kern), F8Big::kLds, lds_set);
  const int64_t blocks = (max_units + kXcds - 1) / kXcds * kXcds + kXcds;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kF8Threads),
                     F8Big::kLds, s, g);
  return hipGetLastError();
}

}  // namespace

GemmPath gemm_path(bool fp8, int64_t rows_per_expert) {
  // Few rows per expert (decode-sized batches): large tiles would spend most
  // of their matrix-core time on padding while the work is weight streaming.
  if (rows_per_expert <= kSkBM) return GEMM_SKINNY;
  if (fp8) return (kF8BM == kBM || rows_per_expert > 2 * kBM) ? GEMM_LARGE_FP8 : GEMM_PIPELINED;
  if (rows_per_expert <= 2 * kBM) return GEMM_PIPELINED;
  // Many rows per expert: 384-row tiles (fewer bytes per FLOP; their
  // padding, a segment's last 129..383 rows, is then a small share).
  return rows_per_expert >= kTallMinRows ? GEMM_LARGE_TALL : GEMM_LARGE;
}

int gemm_path_rows(GemmPath path) {
  switch (path) {
    case GEMM_SKINNY: return kSkBM;
    case GEMM_PIPELINED: return kBM;
    case GEMM_LARGE: return kBigBM;
    case GEMM_LARGE_TALL: return kTallBM;
    case GEMM_LARGE_FP8: return kF8BM;
    case GEMM_MX: return 128;
    case GEMM_MX_LARGE: return 256;
    case GEMM_MX_SKINNY: return kMsBM;
  }
  return kBM;
}

bool gemm_unit_tables(GemmPath path) {
  return path == GEMM_LARGE || path == GEMM_LARGE_TALL || path == GEMM_LARGE_FP8;
}

int gemm_n_tiles(bool swiglu, int Nout) {
  return swiglu ? ceil_div(Nout, kBN / 2) : ceil_div(Nout, kBN);
}

int64_t schedule_entries(int64_t n_pairs, int E_L, GemmPath path, int nt) {
  const int bm = gemm_path_rows(path);
  if (gemm_unit_tables(path)) return (n_pairs / bm + E_L) * nt;
  return ceil_div<int64_t>(n_pairs, bm) + E_L;
}

hipError_t launch_schedule(const int32_t* seg, int seg_cap, int E_L, GemmPath path, int nt_up,
                           int nt_dn, int4* tab_up, int32_t* n_up, int4* tab_dn, int32_t* n_dn,
                           int32_t* sync, int32_t* status, int64_t max_units, hipStream_t s) {
  const int bm = gemm_path_rows(path);
  if (gemm_unit_tables(path)) {  // only the bf16 paths have wide tiles
    // every block redoes the per-expert scan and writes its share of the
    // units (one block wrote some ten thousand entries in 13 us)
    const int64_t want = (max_units + 1023) / 1024;
    const int blocks = static_cast<int>(want < 1 ? 1 : (want > 32 ? 32 : want));
    hipLaunchKernelGGL(unit_schedule_kernel, dim3(blocks), dim3(1024), 0, s, seg, seg_cap, E_L,
                       nt_up, nt_dn, bm, gemm_large_bf16(path), tab_up, n_up, tab_dn, n_dn,
                       status, sync);
  }
  else
    hipLaunchKernelGGL(tile_schedule_kernel, dim3(1), dim3(1024), 0, s, seg, seg_cap, E_L, bm,
                       tab_up, n_up, sync, status);
  return hipGetLastError();
}

// Kernel arguments of one grouped GEMM; hipErrorInvalidValue for requests the
// kernels cannot address.
static hipError_t make_args(const GemmLaunch& L, GemmArgs& g) {
  // The fused gather reads bf16 or E4M3 (block-FP8, MXFP8) row-major
  // sources whose lane offsets fit below the buffer cap.
  static_assert(kGemmGatherMaxBytes <= kBufMax, "gather offsets must stay below the range cap");
  if (L.a_index &&
      (L.a_panel || L.a_rows * (L.fp8 || L.mx ? 1 : 2) * L.K > kGemmGatherMaxBytes))
    return hipErrorInvalidValue;
  g = GemmArgs{};
  g.A = static_cast<const uint8_t*>(L.A);
  g.A_scale = L.A_scale;
  g.W = static_cast<const uint8_t*>(L.W);
  g.W_scale = L.W_scale;
  g.C = L.C;
  g.C_scale = L.C_scale;
  g.seg = L.seg;
  g.seg_cap = L.seg_cap;
  g.info = L.info;
  g.n_tiles = L.n_tiles;
  g.K = L.K;
  g.Nout = L.Nout;
  g.NW = L.swiglu ? 2 * L.Nout : L.Nout;
  g.nt_n = gemm_n_tiles(L.swiglu, L.Nout);
  if (L.mx != (L.path == GEMM_MX || L.path == GEMM_MX_LARGE || L.path == GEMM_MX_SKINNY))
    return hipErrorInvalidValue;
  if (L.mx) {  // E4M3 tokens, E2M1 weights, E8M0 bytes per 32 along K; tokens row
               // major, weights row major or in 128-element panels
    if (L.fp8 || L.a_panel || L.c_panel || L.gelu || L.K % kMxK)
      return hipErrorInvalidValue;
    if (L.swiglu && !L.C_scale) return hipErrorInvalidValue;
    g.w_stride = static_cast<int64_t>(g.NW) * (L.K / 2);
    g.ws_stride = static_cast<int64_t>(g.NW) * (L.K / 32);
    g.a_rs = L.K;
    g.a_cs = 64;
    g.w_rs = L.w_panel ? 64 : L.K / 2;
    g.w_cs = L.w_panel ? 64 * g.NW : 64;
    g.ws_rs = L.w_panel ? 4 : L.K / 32;
    g.ws_cs = L.w_panel ? 4 * g.NW : 4;
    g.a_bytes = L.a_rows * L.K;
    g.a_index = L.a_index;
    return hipSuccess;
  }
  const int64_t elem = L.fp8 ? 1 : 2;
  const int64_t ldb = L.K * elem;
  g.w_stride = static_cast<int64_t>(g.NW) * ldb;
  g.ws_stride = L.fp8 ? static_cast<int64_t>(g.NW / 128) * (L.K / 128) : 0;
  // Per-step buffer offsets are 32-bit: a panel-layout A must span less than
  // the range cap (row-major A is addressed from its tile's first row).
  if (L.a_panel && L.a_rows * ldb > kBufMax) return hipErrorInvalidValue;
  g.a_rs = L.a_panel ? 64 : static_cast<int>(ldb);
  g.a_cs = L.a_panel ? static_cast<int>(64 * L.a_rows) : 64;
  g.w_rs = L.w_panel ? 64 : static_cast<int>(ldb);
  g.w_cs = L.w_panel ? 64 * g.NW : 64;
  g.a_bytes = L.a_rows * ldb;
  g.c_cs = L.c_panel ? 64 * L.c_rows : 0;
  g.a_index = L.a_index;
  g.tickets = L.tickets;
  const bool fp8_path =
      L.path == GEMM_LARGE_FP8 || L.path == GEMM_PIPELINED || L.path == GEMM_SKINNY;
  if ((L.fp8 && !fp8_path) || (!L.fp8 && L.path == GEMM_LARGE_FP8)) return hipErrorInvalidValue;
  if (L.gelu && (L.fp8 || L.swiglu)) return hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_grouped_gemm(const GemmLaunch& L, hipStream_t s) {
  GemmArgs g;
  const hipError_t err = make_args(L, g);
  if (err != hipSuccess) return err;
  switch (L.path) {
    case GEMM_LARGE:
      if (L.gelu) return launch_big<MODE_GELU, kBigBM>(g, L.max_tiles, s);
      return L.swiglu ? launch_big<MODE_SWIGLU, kBigBM>(g, L.max_tiles, s)
                      : launch_big<MODE_PLAIN, kBigBM>(g, L.max_tiles, s);
    case GEMM_LARGE_TALL:
      if (L.gelu) return launch_big<MODE_GELU, kTallBM>(g, L.max_tiles, s);
      return L.swiglu ? launch_big<MODE_SWIGLU, kTallBM>(g, L.max_tiles, s)
                      : launch_big<MODE_PLAIN, kTallBM>(g, L.max_tiles, s);
    case GEMM_SKINNY:
    case GEMM_MX_SKINNY:
      return hipErrorInvalidValue;  // both GEMMs at once: launch_ffn_fused
    case GEMM_MX:
      return L.swiglu ? launch_mx<MODE_SWIGLU_MX8OUT, 128>(g, L.max_tiles, s)
                      : launch_mx<MODE_PLAIN, 128>(g, L.max_tiles, s);
    case GEMM_MX_LARGE:
      return L.swiglu ? launch_mx<MODE_SWIGLU_MX8OUT, 256>(g, L.max_tiles, s)
                      : launch_mx<MODE_PLAIN, 256>(g, L.max_tiles, s);
    case GEMM_LARGE_FP8:
      if (!L.swiglu) return launch_big_fp8<MODE_PLAIN>(g, L.max_tiles, s);
      if (!L.C_scale) return hipErrorInvalidValue;  // block-FP8 h only
      return launch_big_fp8<MODE_SWIGLU_FP8OUT>(g, L.max_tiles, s);
    case GEMM_PIPELINED:
      break;
  }
  if (!L.fp8) {
    if (L.gelu) return launch_pipelined<false, MODE_GELU>(g, L.max_tiles, s);
    return L.swiglu ? launch_pipelined<false, MODE_SWIGLU>(g, L.max_tiles, s)
                    : launch_pipelined<false, MODE_PLAIN>(g, L.max_tiles, s);
  }
  if (L.swiglu) {
    if (L.C_scale) return launch_pipelined<true, MODE_SWIGLU_FP8OUT>(g, L.max_tiles, s);
    return launch_pipelined<true, MODE_SWIGLU>(g, L.max_tiles, s);
  }
  return launch_pipelined<true, MODE_PLAIN>(g, L.max_tiles, s);
}

hipError_t launch_ffn_fused(const GemmLaunch& up, const GemmLaunch& down, int32_t* sync,
                            int32_t* status, hipStream_t s) {
  const bool skinny = up.path == GEMM_SKINNY || up.path == GEMM_MX_SKINNY;
  if (!skinny || down.path != up.path || up.fp8 != down.fp8 || !sync || !status || down.swiglu ||
      down.gelu || up.info != down.info || up.n_tiles != down.n_tiles ||
      up.max_tiles != down.max_tiles)
    return hipErrorInvalidValue;
  GemmArgs gu, gd;
  hipError_t err = make_args(up, gu);
  if (err == hipSuccess) err = make_args(down, gd);
  if (err != hipSuccess) return err;
  if (up.path == GEMM_MX_SKINNY) {  // SwiGLU with MXFP8 h only
    if (!up.swiglu) return hipErrorInvalidValue;
    gd.nt_n = ceil_div(down.Nout, kMsDownBN);  // the down GEMM's wider tiles
    return launch_fused<MODE_SWIGLU_MX8OUT, kSkMx>(gu, gd, up.max_tiles, sync, status, s);
  }
  if (up.fp8) {
    gd.nt_n = ceil_div(down.Nout, sk_down_bn(kSkFp8));  // the down GEMM's wider tiles  // SwiGLU with block-FP8 h only
    if (!up.swiglu || !up.C_scale) return hipErrorInvalidValue;
    return launch_fused<MODE_SWIGLU_FP8OUT, kSkFp8>(gu, gd, up.max_tiles, sync, status, s);
  }
  if (up.gelu) return launch_fused<MODE_GELU, kSkBf16>(gu, gd, up.max_tiles, sync, status, s);
  if (up.swiglu) return launch_fused<MODE_SWIGLU, kSkBf16>(gu, gd, up.max_tiles, sync, status, s);
  return launch_fused<MODE_PLAIN, kSkBf16>(gu, gd, up.max_tiles, sync, status, s);
}

}  // namespace moe
