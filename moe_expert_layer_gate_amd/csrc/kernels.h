// Launchers of the library's kernels (internal; the public ABI is in
// include/moe_layer.h).  Every launcher enqueues on stream `s` and returns
// the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s);

size_t index_scratch_bytes(int T, int E_L);
// cap == 0: contiguous layout (offsets = exclusive scan of counts); cap > 0:
// masked layout, expert e's rows start at e * cap (offsets[e] = e * cap).
hipError_t launch_index_build(const int32_t* topk_ids, int T, int k, int e_lo, int E_L, int cap,
                              int32_t* counts, int32_t* offsets, int32_t* row_token,
                              int32_t* row_slot, int32_t* token_slot_row, void* scratch,
                              hipStream_t s);
constexpr int kIndexFrontMaxTokens = 256;
// The layer's front for 1 <= T <= 256 tokens in one launch: the index build
// of launch_index_build, the m-tile table of the GEMMs without unit tables
// (rows per tile tile_m; sync and status as the schedule kernels take them)
// and, qkind 1 (block-FP8) or 2 (MXFP8), the quantisation of the T rows of
// x [T, H] into xq / xq_scale as launch_gather_fp8 / launch_gather_mx8 with
// the identity map.  hipErrorInvalidValue outside those bounds.
hipError_t launch_index_front(const int32_t* topk_ids, int T, int k, int e_lo, int E_L, int cap,
                              int32_t* counts, int32_t* offsets, int32_t* row_token,
                              int32_t* row_slot, int32_t* token_slot_row, int tile_m, int4* info,
                              int32_t* n_tiles, int32_t* sync, int32_t* status, int qkind,
                              const void* x, int H, void* xq, void* xq_scale, hipStream_t s);
// dst[j] = src[rows[j]] (rows == nullptr: identity) for j < *n_rows, or for
// j < max_rows when n_rows == nullptr.
// With panel_rows > 0, dst is in panel layout [H/32][panel_rows][32].  With
// cap > 0, rows of a masked layout that hold no pair (past counts[e] in expert
// e's block) are skipped.
hipError_t launch_gather_bf16(const void* src, const int32_t* rows, const int32_t* n_rows,
                              int64_t max_rows, int H, void* dst, int64_t panel_rows,
                              hipStream_t s, const int32_t* counts = nullptr, int cap = 0);
// bf16 [batch][rows][cols] row major -> [batch][cols/32][rows][32].
hipError_t launch_pack_panel(const void* src, int64_t batch, int64_t rows, int64_t cols,
                             void* dst, hipStream_t s);
// MX weight scales [batch][rows][cols/32] bytes -> [batch][cols/128][rows][4]
// (cols % 128 == 0).
hipError_t launch_pack_scales_mx(const void* src, int64_t batch, int64_t rows, int64_t cols,
                                 void* dst, hipStream_t s);
hipError_t launch_gather_fp8(const void* src, const int32_t* rows, const int32_t* n_rows,
                             int64_t max_rows, int H, void* dst, float* dst_scale, hipStream_t s,
                             const int32_t* counts = nullptr, int cap = 0);
// MXFP4 conversion of bf16 rows [rows, cols] (cols % 32 == 0): E2M1 codes
// two per byte [rows, cols / 2], E8M0 scales [rows, cols / 32].
hipError_t launch_quant_mx4(const void* src, int64_t rows, int64_t cols, void* codes,
                            uint8_t* scales, hipStream_t s);
// Gather with MXFP8 packing (E4M3 [.., H] + E8M0 [.., H / 32]); arguments as
// launch_gather_fp8.
hipError_t launch_gather_mx8(const void* src, const int32_t* rows, const int32_t* n_rows,
                             int64_t max_rows, int H, void* dst, uint8_t* dst_scale,
                             hipStream_t s, const int32_t* counts = nullptr, int cap = 0);
hipError_t launch_quant_blocks(const void* src, int64_t batch, int64_t rows, int64_t cols,
                               void* codes, float* scales, hipStream_t s);

// GEMM kernels, chosen per problem from the mean rows per expert.
enum GemmPath {
  GEMM_SKINNY = 0,     // bf16 or block-FP8, up to 32 rows: 32 x 256 tiles (decode)
  GEMM_PIPELINED = 1,  // up to 256 rows: 128 x 256 tiles (bf16 and block-FP8)
  GEMM_LARGE = 2,      // bf16: 256 x 256 tiles, 128 x 512 for segment remainders
  GEMM_LARGE_FP8 = 3,  // block-FP8: 256 x 256 tiles
  GEMM_MX = 4,         // MXFP4 weights x MXFP8 activations: 128 x 256 tiles
  GEMM_MX_LARGE = 5,   // the same, more than 256 rows per expert: 256 x 256 tiles
  GEMM_MX_SKINNY = 6,  // the same, up to 32 rows per expert: 32 x 256 tiles (decode)
  GEMM_LARGE_TALL = 7, // bf16, many rows per expert: 384 x 256 tiles, 128 x 512 remainders
};
// The bf16 large-tile paths (per-XCD unit counters, wide remainder tiles).
inline bool gemm_large_bf16(GemmPath path) {
  return path == GEMM_LARGE || path == GEMM_LARGE_TALL;
}
GemmPath gemm_path(bool fp8, int64_t rows_per_expert);
// Token rows of the path's tiles (of its full tiles, for the bf16 large-tile paths).
int gemm_path_rows(GemmPath path);
// Whether the GEMMs run from per-GEMM unit tables (large-tile kernels) or
// from one m-tile table shared by both GEMMs (skinny and pipelined kernels).
bool gemm_unit_tables(GemmPath path);
// n-tiles per expert of one GEMM (every kernel covers 256 weight rows).
int gemm_n_tiles(bool swiglu, int Nout);
// Capacity of a GEMM's work table (nt = gemm_n_tiles of that GEMM) for at
// most n_pairs live rows.
int64_t schedule_entries(int64_t n_pairs, int E_L, GemmPath path, int nt);
// Segment table of the grouped GEMMs: seg_cap == 0: seg = offsets [E_L + 1]
// (contiguous layout, expert e's rows [offsets[e], offsets[e+1])); seg_cap > 0:
// seg = counts [E_L] (masked layout, rows [e seg_cap, e seg_cap + counts[e])).
// Builds the work tables on the device (m-tile table: only tab_up / n_up are
// written).  sync: skinny paths: the fused FFN's ticket and per-m-tile
// counters, [1 + schedule_entries]; large-tile paths: the persistent GEMMs'
// per-XCD unit counters, [kTicketWords] (null: none); cleared here for the
// launches that follow.  status (may be null): the FFN's flag word (kFlag*),
// cleared here.  max_units: the larger table's capacity (schedule_entries).
hipError_t launch_schedule(const int32_t* seg, int seg_cap, int E_L, GemmPath path, int nt_up,
                           int nt_dn, int4* tab_up, int32_t* n_up, int4* tab_dn, int32_t* n_dn,
                           int32_t* sync, int32_t* status, int64_t max_units, hipStream_t s);
// Flag bits of an FFN's status word (the values of MOE_FLAG_* in the ABI).
constexpr int32_t kFlagWaitTimeout = 1;
// Unit counters of the large-tile paths: 8 per GEMM (one per XCD), up then down.
constexpr int kTicketWords = 16;
struct GemmLaunch {
  bool fp8;              // e4m3 operands with block scales, else bf16
  bool mx;               // MXFP4 weights (E2M1, two per byte) x MXFP8 activations,
                         // scales E8M0 bytes per 32 along K (A_scale / W_scale /
                         // C_scale point to bytes); the GEMM_MX* paths
  bool swiglu;           // up GEMM with the SwiGLU epilogue (W = gate and up rows)
  bool gelu;             // up GEMM with the GELU epilogue (bf16); neither: plain
  const void* A;         // [N_cap, K] permuted activations
  const float* A_scale;  // fp8: [N_cap, K/128]
  const void* W;         // [E_L, NW, K]
  const float* W_scale;  // fp8: [E_L, NW/128, K/128]
  void* C;               // [N_cap, Nout]: bf16, or e4m3 when C_scale != nullptr
  float* C_scale;        // fp8 SwiGLU only: [N_cap, Nout/128] per-row group scales
  const int32_t* seg;     // segment table and its layout (see launch_schedule)
  int seg_cap;
  const int4* info;       // work table of this GEMM (launch_schedule)
  const int32_t* n_tiles; // live entries of the table
  int64_t max_tiles;      // its capacity (schedule_entries)
  GemmPath path;          // gemm_path() of the problem
  int K, Nout;
  // Storage layouts (bf16 only): panel = [K/32][R][32], see moe_layer.h.
  bool a_panel;          // A in panel layout with R = a_rows
  bool w_panel;          // each expert's W in panel layout with R = NW
  bool c_panel;          // SwiGLU output h in panel layout with R = c_rows
  int64_t a_rows;        // rows of the A buffer (N_cap, or T with a_index)
  int64_t c_rows;        // rows of the C buffer: N_cap
  // Fused gather (bf16, row-major A only): permuted row j of the GEMM is row
  // a_index[j] of A, e.g. A = the layer input x and a_index = row_token.
  const int32_t* a_index;
  // bf16 large tiles: this GEMM's 8 per-XCD unit counters (from launch_schedule's
  // sync), for the persistent kernel; null runs one block per unit.
  int32_t* tickets;
};
hipError_t launch_grouped_gemm(const GemmLaunch& L, hipStream_t s);
// Both GEMMs of the FFN in one launch (GEMM_SKINNY -- bf16, or block-FP8
// with the SwiGLU up GEMM -- or GEMM_MX_SKINNY with the SwiGLU up GEMM): up
// tiles first, and
// each down tile starts once every up tile of its rows has published h.
// `up` and `down` as for two launch_grouped_gemm calls sharing one m-tile
// table; sync and status as cleared by launch_schedule (a down tile whose
// bounded wait gives up sets kFlagWaitTimeout in *status and is skipped).
hipError_t launch_ffn_fused(const GemmLaunch& up, const GemmLaunch& down, int32_t* sync,
                            int32_t* status, hipStream_t s);
// *flags = OR of the n status words (device pointers), one thread.
hipError_t launch_read_flags(const int32_t* const* words, int n, int32_t* flags, hipStream_t s);
// Largest fused-gather source and largest panel-layout activation matrix
// (bytes) that the GEMM's 32-bit buffer offsets reach.
constexpr int64_t kGemmGatherMaxBytes = 0x7ffffe00;
constexpr int64_t kGemmPanelMaxBytes = 0x7ffffe00;

hipError_t launch_combine(const void* y_perm, const int32_t* token_slot_row, const float* topk_w,
                          const void* shared_out, int T, int k, int H, void* y, hipStream_t s);


}  // namespace moe
