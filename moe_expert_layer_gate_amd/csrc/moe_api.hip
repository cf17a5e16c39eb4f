// Host side of the C ABI declared in include/moe_layer.h: argument checks,
// workspace carving and stage sequencing on the caller's stream.  Nothing here
// allocates device memory or synchronises the host.
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/moe_layer.h"
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

__global__ void fill_offsets_kernel(int32_t* offsets, int n) {
  if (threadIdx.x == 0) {
    offsets[0] = 0;
    offsets[1] = n;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Status words of up to two FFNs (routed and shared expert), by value.
struct FlagWords {
  const int32_t* w[2];
  int n;
};

__global__ void read_flags_kernel(FlagWords words, int32_t* flags) {
  if (threadIdx.x == 0) {
    int32_t f = 0;
    for (int i = 0; i < words.n; ++i) f |= words.w[i][0];
    *flags = f;
  }
}

constexpr int32_t kMaxStreams = 64;  // streams of one streamed layer call

// Validate the problem; returns MOE_OK or MOE_ERR_INVALID_ARG/UNSUPPORTED.
moe_status check_problem(const moe_problem* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  const int64_t T = p->num_tokens, H = p->hidden, E = p->num_experts, k = p->top_k,
                lo = p->expert_begin, EL = p->num_local, I = p->inter, Is = p->shared_inter;
  if (T < 0 || T > (1 << 24)) return MOE_ERR_INVALID_ARG;
  if (E < 1 || E > 1024) return MOE_ERR_INVALID_ARG;
  if (k < 1 || k > E || k > 32) return MOE_ERR_INVALID_ARG;
  if (EL < 1 || EL > 1024 || lo < 0 || lo + EL > E) return MOE_ERR_INVALID_ARG;
  if (H < 128 || H > 65536 || H % 128) return MOE_ERR_INVALID_ARG;
  if (I < 128 || I > 65536 || I % 128) return MOE_ERR_INVALID_ARG;
  if (Is < 0 || Is > 65536 || Is % 128) return MOE_ERR_INVALID_ARG;
  if (p->dtype != MOE_BF16 && p->dtype != MOE_FP8_E4M3 && p->dtype != MOE_MXFP4)
    return MOE_ERR_INVALID_ARG;
  if (p->layout & ~(MOE_LAYOUT_PANEL_WEIGHTS | MOE_LAYOUT_PANEL_ACTS)) return MOE_ERR_INVALID_ARG;
  // block-FP8: row major only; MXFP4: panel weights, row-major activations
  if (p->layout && p->dtype == MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
  if ((p->layout & MOE_LAYOUT_PANEL_ACTS) && p->dtype == MOE_MXFP4) return MOE_ERR_UNSUPPORTED;
  if (p->activation != MOE_ACT_SWIGLU && p->activation != MOE_ACT_GELU) return MOE_ERR_INVALID_ARG;
  if (p->activation == MOE_ACT_GELU && p->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  // One expert's weight matrix must stay below 2 GiB (32-bit buffer offsets).
  if (4 * I * H >= (int64_t(1) << 31) || 4 * Is * H >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  // Masked layout: every expert's block must hold all T tokens; row indices
  // are 32-bit.
  const int64_t C = p->capacity;
  if (C < 0 || C > (1 << 24) || (C > 0 && C < T)) return MOE_ERR_INVALID_ARG;
  if (C * EL >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  // Panel activations: the GEMMs address x_perm and h with 32-bit offsets.
  const int64_t N = C > 0 ? C * EL : T * (k < EL ? k : EL);
  if ((p->layout & MOE_LAYOUT_PANEL_ACTS) && 2 * N * (H > I ? H : I) > kGemmPanelMaxBytes)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Most live (token, local expert) pairs: T min(k, E_L).
int64_t n_pairs(const moe_problem* p) {
  const int64_t kk = p->top_k < p->num_local ? p->top_k : p->num_local;
  return static_cast<int64_t>(p->num_tokens) * kk;
}

// Rows of the permuted buffers: the pairs (contiguous layout) or E_L blocks
// of `capacity` rows (masked layout).
int64_t n_cap(const moe_problem* p) {
  if (p->capacity > 0) return static_cast<int64_t>(p->capacity) * p->num_local;
  return n_pairs(p);
}

bool is_fp8(const moe_problem* p) { return p->dtype == MOE_FP8_E4M3; }
bool is_mx(const moe_problem* p) { return p->dtype == MOE_MXFP4; }
// Quantised GEMM activations with per-row scales (block-FP8 or MXFP8).
bool quant_acts(const moe_problem* p) { return p->dtype != MOE_BF16; }
// Bytes of the activation scales of an [R, C] matrix.
int64_t act_scale_bytes(const moe_problem* p, int64_t R, int64_t C) {
  return is_mx(p) ? R * (C / 32) : 4 * R * (C / 128);
}
bool is_gelu(const moe_problem* p) { return p->activation == MOE_ACT_GELU; }
bool panel_weights(const moe_problem* p) { return p->layout & MOE_LAYOUT_PANEL_WEIGHTS; }
bool panel_acts(const moe_problem* p) { return p->layout & MOE_LAYOUT_PANEL_ACTS; }

// moe_layer's own x_perm and h: panel layout for bf16 whenever the GEMMs can
// address it (the caller's layout bit for activations plays no part).
moe_problem layer_internal(const moe_problem* p) {
  moe_problem q = *p;
  q.layout &= ~MOE_LAYOUT_PANEL_ACTS;
  const int64_t wide = p->hidden > p->inter ? p->hidden : p->inter;
  if (!quant_acts(p) && 2 * n_cap(p) * wide <= kGemmPanelMaxBytes) q.layout |= MOE_LAYOUT_PANEL_ACTS;
  return q;
}

// Bump allocator over the workspace; with base == nullptr it only measures.
struct Carve {
  uint8_t* base;
  size_t used = 0;
  explicit Carve(void* b) : base(static_cast<uint8_t*>(b)) {}
  template <typename T>
  T* take(size_t bytes) {
    used = (used + 255) & ~size_t(255);
    T* r = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += bytes;
    return r;
  }
};

// Fused gather of bf16 sources whose byte size fits the GEMM's 32-bit lane
// offsets.
// The up GEMM can read its rows from the unpermuted tokens (bf16, or the
// E4M3 codes of block-FP8 or MXFP8) through row_token.
bool can_fuse_gather(const moe_problem* p) {
  return static_cast<int64_t>(p->num_tokens) * p->hidden * (quant_acts(p) ? 1 : 2) <=
         kGemmGatherMaxBytes;
}

struct FfnScratch {
  int4* tab_up;     // work tables of the two GEMMs (or one shared m-tile table)
  int4* tab_dn;
  int32_t* n_up;
  int32_t* n_dn;
  int32_t* sync;    // fused decode FFN: ticket + per-m-tile counters
  int32_t* status;  // flag word of the last FFN run on this workspace (MOE_FLAG_*)
  void* h;          // [N_cap, I] bf16 or e4m3
  float* h_scale;   // fp8 only
};

struct FfnShape {
  GemmPath path;
  int nt_up, nt_dn;
  int64_t cap_up, cap_dn;
};

// GEMM kernel family for a mean of `rows` live rows per expert.
GemmPath problem_path(const moe_problem* p, int64_t rows) {
  if (is_mx(p)) return rows > 256 ? GEMM_MX_LARGE : rows > 32 ? GEMM_MX : GEMM_MX_SKINNY;
  return gemm_path(is_fp8(p), rows);
}

// Both GEMMs in one launch (the skinny decode kernels).
bool fused_ffn(GemmPath path) { return path == GEMM_SKINNY || path == GEMM_MX_SKINNY; }

FfnShape ffn_shape(const moe_problem* p) {
  // the kernel family follows the mean live rows per expert, whatever the
  // layout of the buffers
  const int64_t N = n_pairs(p);
  FfnShape f{};
  f.path = problem_path(p, N / p->num_local);
  f.nt_up = gemm_n_tiles(!is_gelu(p), p->inter);
  f.nt_dn = gemm_n_tiles(false, p->hidden);
  f.cap_up = schedule_entries(N, p->num_local, f.path, f.nt_up);
  f.cap_dn = schedule_entries(N, p->num_local, f.path, f.nt_dn);
  return f;
}

FfnScratch carve_ffn(Carve& c, const moe_problem* p) {
  const int64_t N = n_cap(p), I = p->inter;
  const FfnShape sh = ffn_shape(p);
  FfnScratch f{};
  f.status = c.take<int32_t>(sizeof(int32_t));
  f.tab_up = c.take<int4>(sizeof(int4) * sh.cap_up);
  f.n_up = c.take<int32_t>(sizeof(int32_t));
  if (fused_ffn(sh.path)) f.sync = c.take<int32_t>(sizeof(int32_t) * (1 + sh.cap_up));
  if (gemm_large_bf16(sh.path)) f.sync = c.take<int32_t>(sizeof(int32_t) * kTicketWords);
  if (!gemm_unit_tables(sh.path)) {  // one m-tile table for both GEMMs
    f.tab_dn = f.tab_up;
    f.n_dn = f.n_up;
  } else {
    f.tab_dn = c.take<int4>(sizeof(int4) * sh.cap_dn);
    f.n_dn = c.take<int32_t>(sizeof(int32_t));
  }
  if (quant_acts(p)) {
    f.h = c.take<void>(N * I);
    f.h_scale = c.take<float>(act_scale_bytes(p, N, I));
  } else {
    f.h = c.take<void>(2 * N * I);
  }
  return f;
}

struct LayerScratch {
  int32_t* ids;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* row_slot;
  int32_t* tsr;
  void* x_perm;
  float* x_perm_scale;
  void* xq;          // block-FP8 with the fused gather: the tokens quantised
  float* xq_scale;   // once, [T, H] codes and their scales
  void* y_perm;
  void* index_scratch;
  FfnScratch ffn;
  // shared expert
  int32_t* s_offsets;
  void* s_x;
  float* s_x_scale;
  void* s_out;
  FfnScratch s_ffn;
};

moe_problem shared_problem(const moe_problem* p) {
  moe_problem q = *p;
  q.num_experts = 1;
  q.top_k = 1;
  q.expert_begin = 0;
  q.num_local = 1;
  q.inter = p->shared_inter;
  q.shared_inter = 0;
  q.capacity = 0;
  return q;
}

LayerScratch carve_layer(Carve& c, const moe_problem* p) {
  const int64_t T = p->num_tokens, k = p->top_k, EL = p->num_local, H = p->hidden;
  const int64_t N = n_cap(p);
  LayerScratch s{};
  s.ids = c.take<int32_t>(4 * T * k);
  s.w = c.take<float>(4 * T * k);
  s.counts = c.take<int32_t>(4 * EL);
  s.offsets = c.take<int32_t>(4 * (EL + 1));
  s.row_token = c.take<int32_t>(4 * N);
  s.row_slot = c.take<int32_t>(4 * N);
  s.tsr = c.take<int32_t>(4 * T * k);
  // x_perm only where the up GEMM does not gather from the tokens itself;
  // block-FP8 and MX gather from the tokens quantised once
  const bool fuse = can_fuse_gather(p);
  s.x_perm = fuse ? nullptr : c.take<void>((quant_acts(p) ? 1 : 2) * N * H);
  s.x_perm_scale = quant_acts(p) && !fuse ? c.take<float>(act_scale_bytes(p, N, H)) : nullptr;
  if (fuse && quant_acts(p)) {
    s.xq = c.take<void>(T * H);
    s.xq_scale = c.take<float>(act_scale_bytes(p, T, H));
  }
  s.y_perm = c.take<void>(2 * N * H);
  s.index_scratch = c.take<void>(index_scratch_bytes(static_cast<int>(T), static_cast<int>(EL)));
  s.ffn = carve_ffn(c, p);
  if (p->shared_inter > 0) {
    const moe_problem q = shared_problem(p);
    s.s_offsets = c.take<int32_t>(8);
    // the shared expert reads the tokens quantised once (s.xq) whenever the
    // routed experts gather from them; decided on the condition, not on the
    // pointer, which is null while the carve only measures
    if (quant_acts(p) && !fuse) {
      s.s_x = c.take<void>(T * H);
      s.s_x_scale = c.take<float>(act_scale_bytes(p, T, H));
    }
    s.s_out = c.take<void>(2 * T * H);
    s.s_ffn = carve_ffn(c, &q);
  }
  return s;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                                  \
  do {                                                 \
    const hipError_t err__ = (expr);                   \
    if (err__ != hipSuccess) return MOE_ERR_HIP;       \
  } while (0)

// Source rows of the up GEMM (no argument checks):
//   index == nullptr, rows_major == false: x_perm as p->layout says;
//   index == nullptr, rows_major == true:  a row-major [N_cap, H] matrix
//                                          (the shared expert reads x itself);
//   index != nullptr: fused gather, row j is row index[j] of the row-major
//                     [src_rows, H] matrix x (the permutation is never
//                     written out).
struct FfnSource {
  const void* x;
  const float* x_scale;
  bool rows_major;
  const int32_t* index;
  int64_t src_rows;
};

// Enqueue the grouped FFN (no argument checks).  h follows p->layout's
// activation bit.  seg: offsets [E_L + 1], or counts [E_L] when p->capacity
// > 0 (masked layout).  scheduled: the work tables, sync and status were
// already written for these segments (the layer's one-launch front).
moe_status run_ffn(const moe_problem* p, const FfnSource& src, const int32_t* seg,
                   const moe_weights* w, void* h, float* h_scale, void* y_perm,
                   const FfnScratch& f, hipStream_t s, bool scheduled = false) {
  const int64_t N = n_cap(p);
  const int E_L = p->num_local, H = p->hidden, I = p->inter;
  const FfnShape sh = ffn_shape(p);
  void* hb = h ? h : f.h;
  float* hs = h ? h_scale : f.h_scale;
  if (!scheduled)
    MOE_TRY(launch_schedule(seg, p->capacity, E_L, sh.path, sh.nt_up, sh.nt_dn, f.tab_up, f.n_up,
                            f.tab_dn, f.n_dn, f.sync, f.status,
                            sh.cap_up > sh.cap_dn ? sh.cap_up : sh.cap_dn, s));
  GemmLaunch up{};
  up.fp8 = is_fp8(p);
  up.mx = is_mx(p);
  up.swiglu = !is_gelu(p);
  up.gelu = is_gelu(p);
  up.A = src.x;
  up.A_scale = src.x_scale;
  up.W = w->w13;
  up.W_scale = static_cast<const float*>(w->w13_scale);
  up.C = hb;
  up.C_scale = quant_acts(p) ? hs : nullptr;
  up.seg = seg;
  up.seg_cap = p->capacity;
  up.info = f.tab_up;
  up.n_tiles = f.n_up;
  up.max_tiles = sh.cap_up;
  up.path = sh.path;
  up.K = H;
  up.Nout = I;
  up.a_panel = panel_acts(p) && !src.rows_major && !src.index;
  up.w_panel = panel_weights(p);
  up.c_panel = panel_acts(p);
  up.a_rows = src.index ? src.src_rows : N;
  up.c_rows = N;
  up.a_index = src.index;
  up.tickets = gemm_large_bf16(sh.path) ? f.sync : nullptr;
  GemmLaunch down = up;
  down.swiglu = false;
  down.gelu = false;
  down.A = hb;
  down.A_scale = hs;
  down.W = w->w2;
  down.W_scale = static_cast<const float*>(w->w2_scale);
  down.info = f.tab_dn;
  down.n_tiles = f.n_dn;
  down.max_tiles = sh.cap_dn;
  down.C = y_perm;
  down.C_scale = nullptr;
  down.K = I;
  down.Nout = H;
  down.a_panel = panel_acts(p);
  down.c_panel = false;
  down.a_rows = N;
  down.a_index = nullptr;
  down.tickets = gemm_large_bf16(sh.path) ? f.sync + kTicketWords / 2 : nullptr;
  if (fused_ffn(sh.path)) {
    MOE_TRY(launch_ffn_fused(up, down, f.sync, f.status, s));
  } else {
    MOE_TRY(launch_grouped_gemm(up, s));
    MOE_TRY(launch_grouped_gemm(down, s));
  }
  return MOE_OK;
}

// Index build, then (x_perm != nullptr) the gather of the activation rows.
moe_status run_dispatch(const moe_problem* p, const void* x, const int32_t* ids, int32_t* counts,
                        int32_t* offsets, int32_t* row_token, int32_t* row_slot, int32_t* tsr,
                        void* x_perm, float* x_perm_scale, void* scratch, hipStream_t s) {
  const int T = p->num_tokens, E_L = p->num_local, C = p->capacity;
  MOE_TRY(launch_index_build(ids, T, p->top_k, p->expert_begin, E_L, C, counts, offsets,
                             row_token, row_slot, tsr, scratch, s));
  if (!x_perm) return MOE_OK;
  if (is_mx(p))
    MOE_TRY(launch_gather_mx8(x, row_token, offsets + E_L, n_cap(p), p->hidden, x_perm,
                              reinterpret_cast<uint8_t*>(x_perm_scale), s, counts, C));
  else if (is_fp8(p))
    MOE_TRY(launch_gather_fp8(x, row_token, offsets + E_L, n_cap(p), p->hidden, x_perm,
                              x_perm_scale, s, counts, C));
  else
    MOE_TRY(launch_gather_bf16(x, row_token, offsets + E_L, n_cap(p), p->hidden, x_perm,
                               panel_acts(p) ? n_cap(p) : 0, s, counts, C));
  return MOE_OK;
}

bool weights_ok(const moe_problem* p, const moe_weights* w, bool need_shared) {
  if (!w || !w->w13 || !w->w2 || !aligned16(w->w13) || !aligned16(w->w2)) return false;
  if (quant_acts(p) && (!w->w13_scale || !w->w2_scale)) return false;
  if (need_shared) {
    if (!w->ws13 || !w->ws2 || !aligned16(w->ws13) || !aligned16(w->ws2)) return false;
    if (quant_acts(p) && (!w->ws13_scale || !w->ws2_scale)) return false;
  }
  return true;
}

moe_status enqueue_layer(const moe_problem* p, const float* logits, const void* x,
                         const moe_weights* w, void* y, void* ws, hipStream_t s);

// The workspace of moe_layer_static: one array per device, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device memory: kernels get the device address that hipGetSymbolAddress
// returns for the current device, resolved once per device and kept in
// g_scratch (every device holds its own copy of the array).
__device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::atomic<uintptr_t> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's array (resolved on the first call
// on that device).
hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uintptr_t v = g_scratch[dev].load(std::memory_order_acquire);
  if (!v) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    v = g_scratch[dev].load(std::memory_order_relaxed);
    if (!v) {
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255)) return hipErrorInvalidValue;
      v = reinterpret_cast<uintptr_t>(ptr);
      g_scratch[dev].store(v, std::memory_order_release);
    }
  }
  *out = reinterpret_cast<void*>(v);
  return hipSuccess;
}

}  // namespace

hipError_t launch_read_flags(const int32_t* const* words, int n, int32_t* flags, hipStream_t s) {
  if (n < 0 || n > 2) return hipErrorInvalidValue;
  FlagWords fw{};
  for (int i = 0; i < n; ++i) fw.w[i] = words[i];
  fw.n = n;
  hipLaunchKernelGGL(read_flags_kernel, dim3(1), dim3(64), 0, s, fw, flags);
  return hipGetLastError();
}

}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

static void* align_ws(void* ws) {
  const uintptr_t a = (reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255);
  return reinterpret_cast<void*>(a);
}

size_t moe_workspace_bytes(const moe_problem* p, int32_t stage) {
  if (check_problem(p) != MOE_OK) return 0;
  Carve c(nullptr);
  switch (stage) {
    case MOE_STAGE_LAYER: carve_layer(c, p); break;
    case MOE_STAGE_DISPATCH:
      c.take<void>(index_scratch_bytes(p->num_tokens, p->num_local));
      break;
    case MOE_STAGE_FFN: carve_ffn(c, p); break;
    default: return 0;
  }
  return c.used + 256;  // room to round the base up to 256 bytes
}

moe_status moe_workspace_flags(const moe_problem* p, int32_t stage, const void* ws,
                               size_t ws_bytes, int32_t* flags, void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (stage != MOE_STAGE_LAYER && stage != MOE_STAGE_FFN) return MOE_ERR_INVALID_ARG;
  if (!flags || !aligned16(flags)) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe_workspace_bytes(p, stage)) return MOE_ERR_WORKSPACE;
  const int32_t* words[2] = {nullptr, nullptr};
  int n = 0;
  Carve c(align_ws(const_cast<void*>(ws)));
  if (stage == MOE_STAGE_FFN) {
    words[n++] = carve_ffn(c, p).status;
  } else {
    const LayerScratch L = carve_layer(c, p);
    words[n++] = L.ffn.status;
    if (p->shared_inter > 0) words[n++] = L.s_ffn.status;
  }
  return hip_status(launch_read_flags(words, n, flags, static_cast<hipStream_t>(stream)));
}

moe_status moe_route(const moe_problem* p, const float* logits, int32_t* topk_ids,
                     float* topk_w, void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w)) return MOE_ERR_INVALID_ARG;
  if (p->num_tokens == 0) return MOE_OK;
  return hip_status(launch_route_topk(logits, p->num_tokens, p->num_experts, p->top_k, topk_ids,
                                      topk_w, static_cast<hipStream_t>(stream)));
}

moe_status moe_dispatch(const moe_problem* p, const void* x, const int32_t* topk_ids,
                        int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* row_slot,
                        int32_t* token_slot_row, void* x_perm, void* x_perm_scale, void* ws,
                        size_t ws_bytes, void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  const void* ptrs[] = {x, topk_ids, counts, offsets, row_token, row_slot, token_slot_row};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  // x_perm == NULL: index only (the rows are gathered later, e.g. by
  // moe_grouped_ffn_gather)
  if (x_perm && !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  if (x_perm && quant_acts(p) && (!x_perm_scale || !aligned16(x_perm_scale)))
    return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe_workspace_bytes(p, MOE_STAGE_DISPATCH)) return MOE_ERR_WORKSPACE;
  if (p->num_tokens == 0) return MOE_OK;
  // scales: fp32 (block-FP8) or E8M0 bytes (MXFP4); the kernels take either
  // through one float pointer and read it by the element type
  return run_dispatch(p, x, topk_ids, counts, offsets, row_token, row_slot, token_slot_row, x_perm,
                      static_cast<float*>(x_perm_scale), align_ws(ws),
                      static_cast<hipStream_t>(stream));
}

moe_status moe_grouped_ffn(const moe_problem* p, const void* x_perm, const void* x_perm_scale,
                           const int32_t* offsets, const moe_weights* w, void* h, void* h_scale,
                           void* y_perm, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!x_perm || !offsets || !y_perm || !aligned16(x_perm) || !aligned16(offsets) ||
      !aligned16(y_perm))
    return MOE_ERR_INVALID_ARG;
  if (!weights_ok(p, w, false)) return MOE_ERR_INVALID_ARG;
  if (quant_acts(p) && (!x_perm_scale || !aligned16(x_perm_scale))) return MOE_ERR_INVALID_ARG;
  if (h && !aligned16(h)) return MOE_ERR_INVALID_ARG;
  if (h && quant_acts(p) && (!h_scale || !aligned16(h_scale))) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe_workspace_bytes(p, MOE_STAGE_FFN)) return MOE_ERR_WORKSPACE;
  if (p->num_tokens == 0) return MOE_OK;
  Carve c(align_ws(ws));
  const FfnScratch f = carve_ffn(c, p);
  const FfnSource src{x_perm, static_cast<const float*>(x_perm_scale), false, nullptr, 0};
  return run_ffn(p, src, offsets, w, h, static_cast<float*>(h_scale), y_perm, f,
                 static_cast<hipStream_t>(stream));
}

moe_status moe_grouped_ffn_gather(const moe_problem* p, const void* x, const void* x_scale,
                                  const int32_t* row_token, const int32_t* offsets,
                                  const moe_weights* w, void* h, void* h_scale, void* y_perm,
                                  void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!can_fuse_gather(p)) return MOE_ERR_UNSUPPORTED;
  const void* ptrs[] = {x, row_token, offsets, y_perm};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  if (!weights_ok(p, w, false)) return MOE_ERR_INVALID_ARG;
  if (quant_acts(p) && (!x_scale || !aligned16(x_scale))) return MOE_ERR_INVALID_ARG;
  if (h && !aligned16(h)) return MOE_ERR_INVALID_ARG;
  if (h && quant_acts(p) && (!h_scale || !aligned16(h_scale))) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe_workspace_bytes(p, MOE_STAGE_FFN)) return MOE_ERR_WORKSPACE;
  if (p->num_tokens == 0) return MOE_OK;
  Carve c(align_ws(ws));
  const FfnScratch f = carve_ffn(c, p);
  const FfnSource src{x, quant_acts(p) ? static_cast<const float*>(x_scale) : nullptr, true,
                      row_token, p->num_tokens};
  return run_ffn(p, src, offsets, w, h, static_cast<float*>(h_scale), y_perm, f,
                 static_cast<hipStream_t>(stream));
}

moe_status moe_combine(const moe_problem* p, const void* y_perm, const int32_t* token_slot_row,
                       const float* topk_w, const void* shared_out, void* y, void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!y_perm || !token_slot_row || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_perm) || !aligned16(token_slot_row) || !aligned16(topk_w) || !aligned16(y) ||
      (shared_out && !aligned16(shared_out)))
    return MOE_ERR_INVALID_ARG;
  if (p->num_tokens == 0) return MOE_OK;
  return hip_status(launch_combine(y_perm, token_slot_row, topk_w, shared_out, p->num_tokens,
                                   p->top_k, p->hidden, y, static_cast<hipStream_t>(stream)));
}

moe_status moe_layer_static(const moe_problem* p, const float* logits, const void* x,
                            const moe_weights* w, void* y, void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!logits || !x || !y || !aligned16(logits) || !aligned16(x) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  if (!weights_ok(p, w, p->shared_inter > 0)) return MOE_ERR_INVALID_ARG;
  // moe_workspace_bytes adds 256 bytes for rounding a caller's base; the
  // array is 256-byte aligned already
  if (moe_workspace_bytes(p, MOE_STAGE_LAYER) - 256 > MOE_STATIC_SCRATCH_BYTES)
    return MOE_ERR_WORKSPACE;
  if (p->num_tokens == 0) return MOE_OK;
  void* ws = nullptr;
  if (static_scratch(&ws) != hipSuccess) return MOE_ERR_HIP;
  return enqueue_layer(p, logits, x, w, y, ws, static_cast<hipStream_t>(stream));
}

moe_status moe_layer(const moe_problem* p, const float* logits, const void* x,
                     const moe_weights* w, void* y, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!logits || !x || !y || !aligned16(logits) || !aligned16(x) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  if (!weights_ok(p, w, p->shared_inter > 0)) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe_workspace_bytes(p, MOE_STAGE_LAYER)) return MOE_ERR_WORKSPACE;
  if (p->num_tokens == 0) return MOE_OK;
  return enqueue_layer(p, logits, x, w, y, align_ws(ws), static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace moe {
namespace {

// The whole layer on `s` (arguments already checked; ws 256-byte aligned and
// at least moe_workspace_bytes(p, MOE_STAGE_LAYER) - 256 bytes).
moe_status enqueue_layer(const moe_problem* p, const float* logits, const void* x,
                         const moe_weights* w, void* y, void* ws, hipStream_t s) {
  moe_status st = MOE_OK;
  Carve c(ws);
  const LayerScratch L = carve_layer(c, p);
  const int T = p->num_tokens;
  const moe_problem pi = layer_internal(p);

  // The up GEMM gathers its rows from the tokens through row_token, so the
  // permuted activations are never written: bf16 from x, block-FP8 and MX
  // from x quantised once (which the shared expert reads too).
  const bool fuse = can_fuse_gather(p);
  MOE_TRY(launch_route_topk(logits, T, p->num_experts, p->top_k, L.ids, L.w, s));
  // Up to 256 tokens (decode): the index build, the FFN's work table and the
  // quantisation of x in one launch (they share no data).
  const GemmPath path = ffn_shape(&pi).path;
  const bool front = fuse && T <= kIndexFrontMaxTokens && !gemm_unit_tables(path);
  if (front) {
    const int qkind = is_fp8(p) ? 1 : is_mx(p) ? 2 : 0;
    MOE_TRY(launch_index_front(L.ids, T, p->top_k, p->expert_begin, p->num_local, p->capacity,
                               L.counts, L.offsets, L.row_token, L.row_slot, L.tsr,
                               gemm_path_rows(path), L.ffn.tab_up, L.ffn.n_up, L.ffn.sync,
                               L.ffn.status, qkind, x, p->hidden, L.xq, L.xq_scale, s));
  } else {
    st = run_dispatch(&pi, x, L.ids, L.counts, L.offsets, L.row_token, L.row_slot, L.tsr,
                      fuse ? nullptr : L.x_perm, L.x_perm_scale, L.index_scratch, s);
    if (st != MOE_OK) return st;
    if (fuse && is_fp8(p))
      MOE_TRY(launch_gather_fp8(x, nullptr, nullptr, T, p->hidden, L.xq, L.xq_scale, s));
    else if (fuse && is_mx(p))
      MOE_TRY(launch_gather_mx8(x, nullptr, nullptr, T, p->hidden, L.xq,
                                reinterpret_cast<uint8_t*>(L.xq_scale), s));
  }
  const void* xa = x;
  const float* xa_scale = nullptr;
  if (fuse && quant_acts(p)) {
    xa = L.xq;
    xa_scale = L.xq_scale;
  }
  const FfnSource rsrc = fuse ? FfnSource{xa, xa_scale, true, L.row_token, T}
                              : FfnSource{L.x_perm, L.x_perm_scale, false, nullptr, 0};
  st = run_ffn(&pi, rsrc, p->capacity > 0 ? L.counts : L.offsets, w, nullptr, nullptr, L.y_perm,
               L.ffn, s, front);
  if (st != MOE_OK) return st;
  if (p->shared_inter > 0) {
    const moe_problem sq = shared_problem(p);
    const moe_problem q = layer_internal(&sq);
    moe_weights sw{};
    sw.w13 = w->ws13;
    sw.w2 = w->ws2;
    sw.w13_scale = w->ws13_scale;
    sw.w2_scale = w->ws2_scale;
    hipLaunchKernelGGL(fill_offsets_kernel, dim3(1), dim3(64), 0, s, L.s_offsets, T);
    MOE_TRY(hipGetLastError());
    const void* sx = x;
    const float* sx_scale = nullptr;
    if (L.xq) {
      sx = L.xq;
      sx_scale = L.xq_scale;
    } else if (is_mx(p)) {
      MOE_TRY(launch_gather_mx8(x, nullptr, nullptr, T, p->hidden, L.s_x,
                                reinterpret_cast<uint8_t*>(L.s_x_scale), s));
      sx = L.s_x;
      sx_scale = L.s_x_scale;
    } else if (is_fp8(p)) {
      MOE_TRY(launch_gather_fp8(x, nullptr, nullptr, T, p->hidden, L.s_x, L.s_x_scale, s));
      sx = L.s_x;
      sx_scale = L.s_x_scale;
    }
    const FfnSource ssrc{sx, sx_scale, true, nullptr, 0};
    st = run_ffn(&q, ssrc, L.s_offsets, &sw, nullptr, nullptr, L.s_out, L.s_ffn, s);
    if (st != MOE_OK) return st;
  }
  return hip_status(launch_combine(L.y_perm, L.tsr, L.w, p->shared_inter > 0 ? L.s_out : nullptr,
                                   T, p->top_k, p->hidden, y, s));
}

}  // namespace
}  // namespace moe

extern "C" {

moe_status moe_quantize_fp8(const void* src, int64_t batch, int64_t rows, int64_t cols,
                            int32_t block_rows, void* codes, float* scales, void* stream) {
  if (!src || !codes || !scales || !aligned16(src) || !aligned16(codes) || !aligned16(scales))
    return MOE_ERR_INVALID_ARG;
  if (batch < 0 || rows < 0 || cols < 128 || cols % 128 || cols > (1 << 20))
    return MOE_ERR_INVALID_ARG;
  if (block_rows != 1 && block_rows != 128) return MOE_ERR_INVALID_ARG;
  if (batch * rows > (int64_t(1) << 31) - 1) return MOE_ERR_INVALID_ARG;
  if (batch == 0 || rows == 0) return MOE_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (block_rows == 1) {
    if (cols > 65536) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_gather_fp8(src, nullptr, nullptr, batch * rows,
                                        static_cast<int>(cols), codes, scales, s));
  }
  if ((rows + 127) / 128 > 65535 || batch > 65535) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quant_blocks(src, batch, rows, cols, codes, scales, s));
}

moe_status moe_quantize_mx(const void* src, int64_t batch, int64_t rows, int64_t cols,
                           int32_t elem, void* codes, void* scales, void* stream) {
  if (!src || !codes || !scales || !aligned16(src) || !aligned16(codes) || !aligned16(scales))
    return MOE_ERR_INVALID_ARG;
  if (batch < 0 || rows < 0 || cols < 32 || cols % 32 || cols > (1 << 20))
    return MOE_ERR_INVALID_ARG;
  if (elem != MOE_MX_E2M1 && elem != MOE_MX_E4M3) return MOE_ERR_INVALID_ARG;
  if (batch * rows > (int64_t(1) << 31) - 1) return MOE_ERR_INVALID_ARG;
  if (batch == 0 || rows == 0) return MOE_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (elem == MOE_MX_E2M1)
    return hip_status(launch_quant_mx4(src, batch * rows, cols, codes,
                                       static_cast<uint8_t*>(scales), s));
  if (cols % 128 || cols > 65536) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_gather_mx8(src, nullptr, nullptr, batch * rows, static_cast<int>(cols),
                                      codes, static_cast<uint8_t*>(scales), s));
}

moe_status moe_pack_panel(const void* src, int64_t batch, int64_t rows, int64_t cols, void* dst,
                          void* stream) {
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return MOE_ERR_INVALID_ARG;
  if (batch < 0 || rows < 0 || cols < 32 || cols % 32 || cols > (1 << 20))
    return MOE_ERR_INVALID_ARG;
  if (rows > 0 && batch > ((int64_t(1) << 40) / cols) / rows) return MOE_ERR_INVALID_ARG;
  const int64_t bytes = 2 * batch * rows * cols;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (bytes > 0 && a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARG;
  if (batch == 0 || rows == 0) return MOE_OK;
  return hip_status(launch_pack_panel(src, batch, rows, cols, dst, static_cast<hipStream_t>(stream)));
}

moe_status moe_pack_panel_mx(const void* codes, const void* scales, int64_t batch, int64_t rows,
                             int64_t cols, void* codes_dst, void* scales_dst, void* stream) {
  const void* ptrs[] = {codes, scales, codes_dst, scales_dst};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  if (batch < 0 || rows < 0 || cols < 128 || cols % 128 || cols > (1 << 20))
    return MOE_ERR_INVALID_ARG;
  if (rows > 0 && batch > ((int64_t(1) << 40) / cols) / rows) return MOE_ERR_INVALID_ARG;
  const int64_t cb = batch * rows * (cols / 2), sb = batch * rows * (cols / 32);
  auto overlap = [](const void* x, int64_t nx, const void* y, int64_t ny) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    return nx > 0 && ny > 0 && a < b + ny && b < a + nx;
  };
  if (overlap(codes, cb, codes_dst, cb) || overlap(codes, cb, scales_dst, sb) ||
      overlap(scales, sb, codes_dst, cb) || overlap(scales, sb, scales_dst, sb) ||
      overlap(codes_dst, cb, scales_dst, sb))
    return MOE_ERR_INVALID_ARG;
  if (batch == 0 || rows == 0) return MOE_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the code bytes of a row are cols / 4 two-byte units: bf16 panels of 32
  // units are the 64-byte (128-element) MX panels
  MOE_TRY(launch_pack_panel(codes, batch, rows, cols / 4, codes_dst, s));
  return hip_status(launch_pack_scales_mx(scales, batch, rows, cols, scales_dst, s));
}

// ---------------------------------------------------------------------------
// Streaming FFN (page "CascadeEP ...", section 3.2 and Appendix C): the host
// side of the launch threshold and of threshold batching, and the streamed
// layer that runs each invocation on its own stream.
// ---------------------------------------------------------------------------

int64_t moe_stream_threshold(const int64_t* counts, const double* throughput, int32_t n,
                             double rho) {
  if (!counts || !throughput || n < 1 || !(rho >= 0.0 && rho <= 1.0)) return -1;
  double peak = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    if (!(throughput[i] >= 0.0) || throughput[i] > 1e300 || counts[i] < 0) return -1;
    if (throughput[i] > peak) peak = throughput[i];
  }
  int64_t best = -1;
  for (int32_t i = 0; i < n; ++i)
    if (throughput[i] >= rho * peak && (best < 0 || counts[i] < best)) best = counts[i];
  return best;
}

moe_status moe_stream_plan(const int64_t* ready_rows, int32_t n, int64_t theta,
                           int32_t* group_end, int32_t* n_groups) {
  if (!n_groups || n < 0 || theta < 0 || (n > 0 && (!ready_rows || !group_end)))
    return MOE_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (ready_rows[i] < 0) return MOE_ERR_INVALID_ARG;
  int32_t g = 0;
  int64_t pending = 0;
  for (int32_t i = 0; i < n; ++i) {
    pending += ready_rows[i];
    if (pending >= theta || i == n - 1) {  // threshold reached, or the final flush
      group_end[g++] = i + 1;
      pending = 0;
    }
  }
  *n_groups = g;
  return MOE_OK;
}

// Workspace of one stream's slice: enough for the layer on any group of up to
// max_group_tokens tokens.  Within one GEMM path the layer's workspace grows
// with the token count, but the work tables change form where the path does,
// so the largest count of every smaller path is measured too.
static size_t streamed_slice(const moe_problem* p, int32_t max_group_tokens) {
  moe_problem q = *p;
  q.num_tokens = max_group_tokens;
  size_t b = moe_workspace_bytes(&q, MOE_STAGE_LAYER);
  const int64_t kk = p->top_k < p->num_local ? p->top_k : p->num_local;
  for (int64_t r = 0; r < 4096; ++r) {
    if (problem_path(p, r) == problem_path(p, r + 1)) continue;
    // routed experts: rows per expert T kk / E_L; the shared expert: T
    const int64_t cands[2] = {((r + 1) * p->num_local - 1) / kk, r};
    for (const int64_t t : cands) {
      if (t <= 0 || t >= max_group_tokens) continue;
      q.num_tokens = static_cast<int32_t>(t);
      const size_t bt = moe_workspace_bytes(&q, MOE_STAGE_LAYER);
      if (bt > b) b = bt;
    }
  }
  return (b + 255) & ~size_t(255);
}

size_t moe_workspace_bytes_streamed(const moe_problem* p, int32_t max_group_tokens,
                                    int32_t n_streams) {
  if (check_problem(p) != MOE_OK || max_group_tokens < 0 ||
      max_group_tokens > p->num_tokens || n_streams < 1 || n_streams > kMaxStreams)
    return 0;
  return streamed_slice(p, max_group_tokens) * static_cast<size_t>(n_streams);
}

moe_status moe_layer_streamed(const moe_problem* p, const float* logits, const void* x,
                              const moe_weights* w, void* y, const int32_t* group_tokens,
                              int32_t n_groups, void* const* streams, int32_t n_streams,
                              void* ws, size_t ws_bytes) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!logits || !x || !y || !aligned16(logits) || !aligned16(x) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  if (!weights_ok(p, w, p->shared_inter > 0)) return MOE_ERR_INVALID_ARG;
  if (!streams || n_streams < 1 || n_streams > kMaxStreams || n_groups < 0 || !group_tokens)
    return MOE_ERR_INVALID_ARG;
  // group_tokens: 0 = g_0 <= g_1 <= ... <= g_n = T
  if (group_tokens[0] != 0 || group_tokens[n_groups] != p->num_tokens) return MOE_ERR_INVALID_ARG;
  int32_t max_g = 0;
  for (int32_t j = 0; j < n_groups; ++j) {
    const int32_t len = group_tokens[j + 1] - group_tokens[j];
    if (len < 0) return MOE_ERR_INVALID_ARG;
    if (len > max_g) max_g = len;
  }
  const size_t slice = streamed_slice(p, max_g);
  if (!ws || ws_bytes < slice * static_cast<size_t>(n_streams)) return MOE_ERR_WORKSPACE;
  uint8_t* base = static_cast<uint8_t*>(align_ws(ws));
  // the 256 bytes of slack in each slice absorb the base's rounding
  const int64_t E = p->num_experts, H = p->hidden;
  for (int32_t j = 0; j < n_groups; ++j) {
    const int32_t t0 = group_tokens[j], len = group_tokens[j + 1] - t0;
    if (len == 0) continue;
    moe_problem q = *p;
    q.num_tokens = len;
    const int32_t si = j % n_streams;
    st = enqueue_layer(&q, logits + t0 * E, static_cast<const uint16_t*>(x) + t0 * H, w,
                       static_cast<uint16_t*>(y) + t0 * H, base + si * slice,
                       static_cast<hipStream_t>(streams[si]));
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

}  // extern "C"
