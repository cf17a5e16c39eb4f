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
// Tile schedule: one block turns the device-resident expert offsets into a
// list of 128-row m-tiles (expert, first row, end row) -- ceil(n_e / 128)
// tiles per expert, none for an empty expert -- plus their count.  The GEMM
// grid is (n-tiles, upper bound of m-tiles) and blocks past the live count
// exit at once, so no host sync is needed for the data-dependent sizes.
//
// Block tile: 128 token rows x 128 weight rows x K-step, 4 waves in a 2 x 2
// arrangement, each wave 64 x 64 as 2 x 2 MFMA 32x32 tiles.  The weight tile is
// the MFMA A operand and the token tile the B operand, so each lane's
// accumulator holds 4 consecutive output columns of one token row (one 8-byte
// store).  Operands are staged through LDS (row pitch padded by 16 bytes,
// which spreads the 16-byte fragment reads of 16 consecutive rows over all
// banks) with double buffering: the global loads of step k+1 are in flight
// while step k computes.
//
// SwiGLU mode: the 128 weight rows of a block are 64 gate rows and the 64
// matching up rows, arranged so each wave holds gate and up accumulators for
// the same (row, column) in the same lane; the epilogue writes
// h = silu(gate) * up and never materialises the [n, 2I] product.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kBM = 128;   // token rows per block
constexpr int kBN = 128;   // weight rows per block
constexpr int kBKb = 128;  // bytes of K per step (64 bf16 or 128 fp8)
constexpr int kPitch = kBKb + 16;  // LDS row pitch in bytes

__global__ __launch_bounds__(1024) void tile_schedule_kernel(
    const int32_t* __restrict__ offsets, int E_L, int4* __restrict__ info,
    int32_t* __restrict__ n_tiles) {
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E_L) cnt = offsets[e + 1] - offsets[e];
  const int tiles = ceil_div(cnt, kBM);
  int total;
  const int start = block_exclusive_scan(tiles, &total);
  if (e < E_L) {
    const int r0 = offsets[e], r1 = offsets[e + 1];
    for (int i = 0; i < tiles; ++i) info[start + i] = make_int4(e, r0 + i * kBM, r1, 0);
  }
  if (e == 0) *n_tiles = total;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// Global -> register -> LDS staging of one K-step of the two operand tiles.
// Thread `tid` moves 16-byte chunks c = tid + 256 i (i < 4) of each tile:
// row c / 8, byte column (c % 8) * 16.
struct TileLoader {
  const uint8_t* gW[4];
  const uint8_t* gA[4];
  int sOff[4];
  uint4 rW[4], rA[4];

  __device__ __forceinline__ void init(const uint8_t* We, const uint8_t* A, int64_t ldw,
                                       int64_t lda, int nt, int Nout, bool swiglu, int row0,
                                       int row_end) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3, col = (c & 7) * 16;
      const int wrow = swiglu ? (r < 64 ? nt * 64 + r : Nout + nt * 64 + (r - 64)) : nt * kBN + r;
      gW[i] = We + static_cast<int64_t>(wrow) * ldw + col;
      const int arow = min(row0 + r, row_end - 1);
      gA[i] = A + static_cast<int64_t>(arow) * lda + col;
      sOff[i] = r * kPitch + col;
    }
  }
  __device__ __forceinline__ void load(int64_t kbyte) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rW[i] = *reinterpret_cast<const uint4*>(gW[i] + kbyte);
      rA[i] = *reinterpret_cast<const uint4*>(gA[i] + kbyte);
    }
  }
  __device__ __forceinline__ void store(uint8_t* sW, uint8_t* sA) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(sW + sOff[i]) = rW[i];
      *reinterpret_cast<uint4*>(sA + sOff[i]) = rA[i];
    }
  }
};

// LDS row of the wave's weight block i (0, 1) and token block j (0, 1).
__device__ __forceinline__ int wrow_of(bool swiglu, int wn, int i) {
  return swiglu ? (i == 0 ? wn * 32 : 64 + wn * 32) : wn * 64 + i * 32;
}

template <bool SWIGLU>
__global__ __launch_bounds__(256, 2) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, uint16_t* __restrict__ C,
    const int4* __restrict__ info, const int32_t* __restrict__ n_tiles, int K, int Nout,
    int64_t w_expert_stride) {
  __shared__ __attribute__((aligned(16))) uint8_t sW[2][kBN * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kBM * kPitch];
  const int mt = blockIdx.y;
  if (mt >= *n_tiles) return;
  const int4 ti = info[mt];
  const int e = ti.x, row0 = ti.y, row_end = ti.z;
  const int nt = blockIdx.x;

  TileLoader ld;
  ld.init(reinterpret_cast<const uint8_t*>(W + e * w_expert_stride),
          reinterpret_cast<const uint8_t*>(A), 2ll * K, 2ll * K, nt, Nout, SWIGLU, row0, row_end);

  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int lr = lane & 31, kq = (lane >> 5) * 16;  // byte offset of the lane's 8 k values
  int offW[2], offA[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) offW[i] = (wrow_of(SWIGLU, wn, i) + lr) * kPitch + kq;
#pragma unroll
  for (int j = 0; j < 2; ++j) offA[j] = (wm * 64 + j * 32 + lr) * kPitch + kq;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (2 * K) / kBKb;
  ld.load(0);
  ld.store(sW[0], sA[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) ld.load(static_cast<int64_t>(kt + 1) * kBKb);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {  // 4 x 16 bf16 = 64 k per step
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const bf16x8*>(&sW[buf][offW[i] + kk * 32]);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const bf16x8*>(&sA[buf][offA[j] + kk * 32]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) ld.store(sW[buf ^ 1], sA[buf ^ 1]);
    __syncthreads();
  }

  // Epilogue.  Accumulator element g*4 + r of a 32x32 tile is weight row
  // g*8 + (lane/32)*4 + r and token row lane%32.
  const int cq = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = row0 + wm * 64 + j * 32 + lr;
    if (m >= row_end) continue;
    uint16_t* crow = C + static_cast<int64_t>(m) * Nout;
    if (SWIGLU) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[r] = silu_mul(acc[0][j][g * 4 + r], acc[1][j][g * 4 + r]);
        uint2 o;
        o.x = pack_bf16x2(hv[0], hv[1]);
        o.y = pack_bf16x2(hv[2], hv[3]);
        *reinterpret_cast<uint2*>(crow + nt * 64 + wn * 32 + g * 8 + cq) = o;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 o;
          o.x = pack_bf16x2(acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1]);
          o.y = pack_bf16x2(acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]);
          *reinterpret_cast<uint2*>(crow + nt * kBN + wn * 64 + i * 32 + g * 8 + cq) = o;
        }
    }
  }
}

// Block-FP8 version: E4M3 operands, one K-step = one 128-wide scale block.
// Each step's two MFMA 32x32x64 products go to a zeroed temporary which is
// added to the accumulator times (weight block scale x token group scale).
// Output is bf16 (h before its own quantisation, or y).
template <bool SWIGLU>
__global__ __launch_bounds__(256, 2) void grouped_gemm_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ A_scale,
    const uint8_t* __restrict__ W, const float* __restrict__ W_scale, uint16_t* __restrict__ C,
    const int4* __restrict__ info, const int32_t* __restrict__ n_tiles, int K, int Nout,
    int64_t w_expert_stride, int64_t ws_expert_stride) {
  __shared__ __attribute__((aligned(16))) uint8_t sW[2][kBN * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kBM * kPitch];
  const int mt = blockIdx.y;
  if (mt >= *n_tiles) return;
  const int4 ti = info[mt];
  const int e = ti.x, row0 = ti.y, row_end = ti.z;
  const int nt = blockIdx.x;
  const int kb_n = K / 128;

  TileLoader ld;
  ld.init(W + e * w_expert_stride, A, K, K, nt, Nout, SWIGLU, row0, row_end);

  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int lr = lane & 31, kq = (lane >> 5) * 32;  // byte offset of the lane's 32 k values
  int offW[2], offA[2];
  const float* sWrow[2];
  const float* sArow[2];
  const float* wsc = W_scale + e * ws_expert_stride;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int lrow = wrow_of(SWIGLU, wn, i);
    offW[i] = (lrow + lr) * kPitch + kq;
    const int grow = SWIGLU ? (lrow < 64 ? nt * 64 + lrow : Nout + nt * 64 + (lrow - 64))
                            : nt * kBN + lrow;
    sWrow[i] = wsc + static_cast<int64_t>(grow / 128) * kb_n;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    offA[j] = (wm * 64 + j * 32 + lr) * kPitch + kq;
    const int arow = min(row0 + wm * 64 + j * 32 + lr, row_end - 1);
    sArow[j] = A_scale + static_cast<int64_t>(arow) * kb_n;
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  ld.load(0);
  ld.store(sW[0], sA[0]);
  __syncthreads();
  for (int kt = 0; kt < kb_n; ++kt) {
    const int buf = kt & 1;
    float sw[2], sx[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) sw[i] = sWrow[i][kt];
#pragma unroll
    for (int j = 0; j < 2; ++j) sx[j] = sArow[j][kt];
    if (kt + 1 < kb_n) ld.load(static_cast<int64_t>(kt + 1) * kBKb);
    f32x16 tmp[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmp[i][j][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {  // 2 x 64 fp8 = 128 k per step
      i32x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(&sW[buf][offW[i] + kk * 64]);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(&sW[buf][offW[i] + kk * 64 + 16]);
        a[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(&sA[buf][offA[j] + kk * 64]);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(&sA[buf][offA[j] + kk * 64 + 16]);
        b[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          tmp[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], tmp[i][j], 0, 0,
                                                                      0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float sc = sw[i] * sx[j];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] += tmp[i][j][r] * sc;
      }
    if (kt + 1 < kb_n) ld.store(sW[buf ^ 1], sA[buf ^ 1]);
    __syncthreads();
  }

  const int cq = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = row0 + wm * 64 + j * 32 + lr;
    if (m >= row_end) continue;
    uint16_t* crow = C + static_cast<int64_t>(m) * Nout;
    if (SWIGLU) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[r] = silu_mul(acc[0][j][g * 4 + r], acc[1][j][g * 4 + r]);
        uint2 o;
        o.x = pack_bf16x2(hv[0], hv[1]);
        o.y = pack_bf16x2(hv[2], hv[3]);
        *reinterpret_cast<uint2*>(crow + nt * 64 + wn * 32 + g * 8 + cq) = o;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 o;
          o.x = pack_bf16x2(acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1]);
          o.y = pack_bf16x2(acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]);
          *reinterpret_cast<uint2*>(crow + nt * kBN + wn * 64 + i * 32 + g * 8 + cq) = o;
        }
    }
  }
}

}  // namespace

int64_t max_m_tiles(int64_t n_cap, int E_L) { return ceil_div<int64_t>(n_cap, kBM) + E_L; }

hipError_t launch_tile_schedule(const int32_t* offsets, int E_L, int4* info, int32_t* n_tiles,
                                hipStream_t s) {
  hipLaunchKernelGGL(tile_schedule_kernel, dim3(1), dim3(1024), 0, s, offsets, E_L, info, n_tiles);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(bool swiglu, const void* A, const void* W, void* C, const int4* info,
                            const int32_t* n_tiles, int64_t max_tiles, int K, int Nout,
                            int64_t w_expert_stride, hipStream_t s) {
  const int ntn = swiglu ? Nout / 64 : Nout / kBN;
  const dim3 grid(ntn, static_cast<unsigned>(max_tiles)), block(256);
  if (swiglu)
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<true>, grid, block, 0, s,
                       static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(W),
                       static_cast<uint16_t*>(C), info, n_tiles, K, Nout, w_expert_stride);
  else
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<false>, grid, block, 0, s,
                       static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(W),
                       static_cast<uint16_t*>(C), info, n_tiles, K, Nout, w_expert_stride);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(bool swiglu, const void* A, const float* A_scale, const void* W,
                           const float* W_scale, void* C, const int4* info,
                           const int32_t* n_tiles, int64_t max_tiles, int K, int Nout,
                           int64_t w_expert_stride, int64_t ws_expert_stride, hipStream_t s) {
  const int ntn = swiglu ? Nout / 64 : Nout / kBN;
  const dim3 grid(ntn, static_cast<unsigned>(max_tiles)), block(256);
  if (swiglu)
    hipLaunchKernelGGL(grouped_gemm_fp8_kernel<true>, grid, block, 0, s,
                       static_cast<const uint8_t*>(A), A_scale, static_cast<const uint8_t*>(W),
                       W_scale, static_cast<uint16_t*>(C), info, n_tiles, K, Nout,
                       w_expert_stride, ws_expert_stride);
  else
    hipLaunchKernelGGL(grouped_gemm_fp8_kernel<false>, grid, block, 0, s,
                       static_cast<const uint8_t*>(A), A_scale, static_cast<const uint8_t*>(W),
                       W_scale, static_cast<uint16_t*>(C), info, n_tiles, K, Nout,
                       w_expert_stride, ws_expert_stride);
  return hipGetLastError();
}

}  // namespace moe
