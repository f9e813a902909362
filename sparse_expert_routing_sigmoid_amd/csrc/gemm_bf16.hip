// Grouped SwiGLU expert GEMMs on bf16 MFMA (gfx950) and a plain fp32 path.
//
// The FFN of every expert in the combine equation of the "DeepSeek-V3
// Technical Report" reading guide (xyznot.com, Method section 2).  The pages
// do not print the FFN form; this library uses SwiGLU:
//   h = SiLU(x W_gate^T) * (x W_up^T),   y = h W_down^T.
//
// Phase A (k_gateup_*): for every row tile of a segment, gathers the token
// rows of x through row_token, multiplies by the expert's gate and up rows
// together, and applies SwiGLU in the epilogue, so only h ([P, I], bf16)
// goes back to HBM.  Phase B (k_down_*): y = h W_down^T for the same tiles.
//
// Tiling (bf16): 256 threads = 4 waves as 2 x 2; block tile 128 rows x 128
// weight rows x 64 K; every wave owns 64 rows x 64 weight rows as 2 x 2
// 32x32x16 MFMA tiles with fp32 accumulators.  Operands are staged through
// LDS (rows padded by 16 B against bank conflicts) with register
// double buffering of the next K slab.  In phase A a wave's weight rows are
// 32 gate rows and the 32 up rows of the same h columns, so SwiGLU pairs
// accumulators that sit in the same lane and register.
#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int BM = 128;
constexpr int BN = 128;  // weight rows per block
constexpr int BK = 64;
constexpr int LDA = BK + 8;  // padded LDS row, in bf16 elements
constexpr int NTHR = 256;

struct TileInfo {
  int seg, row0, rows;
  bool live;
};

// Block -> (tile of the map, 128-row half of it).  Tiles hold up to 256 rows.
__device__ __forceinline__ TileInfo tile_of_block(const int32_t* tile_map, const int32_t* n_tiles, int bx) {
  TileInfo ti;
  const int tile = bx >> 1;
  const int half = bx & 1;
  ti.live = false;
  ti.seg = ti.row0 = ti.rows = 0;
  if (tile >= *n_tiles) return ti;
  const int4 m = *reinterpret_cast<const int4*>(tile_map + 4LL * tile);
  const int r = m.z - half * BM;
  if (r <= 0) return ti;
  ti.live = true;
  ti.seg = m.x;
  ti.row0 = m.y + half * BM;
  ti.rows = r < BM ? r : BM;
  return ti;
}


// Loads one 128 x 64 bf16 slab (4 x 16 B per thread) from row pointers.
struct Slab {
  uint4 v[4];
};

__device__ __forceinline__ void slab_load(Slab& s, const uint16_t* const (&src)[4], int k0) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (src[i])
      s.v[i] = *reinterpret_cast<const uint4*>(src[i] + k0);
    else
      s.v[i] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void slab_store(uint16_t* lds, const Slab& s, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + NTHR * i;
    const int r = c >> 3, ch = c & 7;
    *reinterpret_cast<uint4*>(lds + r * LDA + ch * 8) = s.v[i];
  }
}

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t* lds, int row, int kofs) {
  const uint4 q = *reinterpret_cast<const uint4*>(lds + row * LDA + kofs);
  return __builtin_bit_cast(bf16x8_t, q);
}

// Core: C[2][2] (each 32x32) += A(rows am0..am0+63) * B(rows bn[0], bn[1])^T
// over one 64-wide K slab held in LDS.
__device__ __forceinline__ void mma_slab(f32x16_t (&acc)[2][2], const uint16_t* la, const uint16_t* lb, int am0,
                                         const int (&bn)[2], int lane) {
  const int r = lane & 31;
  const int kg = (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < BK; kk += 16) {
    bf16x8_t a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = lds_frag(la, am0 + i * 32 + r, kk + kg);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = lds_frag(lb, bn[j] + r, kk + kg);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Accumulator element (i of 16) of a 32x32 tile: row and column inside it.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

__global__ __launch_bounds__(NTHR) void k_gateup_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w13,
                                                      const int32_t* __restrict__ row_token,
                                                      const int32_t* __restrict__ tile_map,
                                                      const int32_t* __restrict__ n_tiles, int d, int I,
                                                      uint16_t* __restrict__ h) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][BM * LDA];
  const TileInfo ti = tile_of_block(tile_map, n_tiles, blockIdx.x);
  if (!ti.live) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int c0 = blockIdx.y * (BN / 2);  // first h column of the block
  const uint16_t* wexp = w13 + (long long)ti.seg * 2 * I * d;

  const uint16_t* asrc[4];
  const uint16_t* bsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + NTHR * i;
    const int r = c >> 3, ch = c & 7;
    int tok = -1;
    if (r < ti.rows) tok = row_token[ti.row0 + r];
    asrc[i] = tok >= 0 ? x + (long long)tok * d + ch * 8 : nullptr;
    // weight rows 0..63 of the tile: gate rows c0.., 64..127: up rows I+c0..
    const int wrow = r < BN / 2 ? c0 + r : I + c0 + (r - BN / 2);
    bsrc[i] = wexp + (long long)wrow * d + ch * 8;
  }

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  Slab sa, sb;
  slab_load(sa, asrc, 0);
  slab_load(sb, bsrc, 0);
  slab_store(lds[0][0], sa, tid);
  slab_store(lds[0][1], sb, tid);
  __syncthreads();
  const int nk = d / BK;
  const int bn[2] = {wn * 32, BN / 2 + wn * 32};  // gate rows, up rows of this wave
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      slab_load(sa, asrc, (kt + 1) * BK);
      slab_load(sb, bsrc, (kt + 1) * BK);
    }
    mma_slab(acc, lds[cur][0], lds[cur][1], wm * 64, bn, lane);
    if (kt + 1 < nk) {
      slab_store(lds[cur ^ 1][0], sa, tid);
      slab_store(lds[cur ^ 1][1], sb, tid);
    }
    __syncthreads();
  }
  // Epilogue: h = SiLU(gate) * up, rounded to bf16.
  const int col = c0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = wm * 64 + i * 32 + acc_row(e, lane);
      if (r < ti.rows) {
        const float v = silu(acc[i][0][e]) * acc[i][1][e];
        h[(long long)(ti.row0 + r) * I + col] = f32_to_bf16(v);
      }
    }
}

template <typename YT>
__device__ __forceinline__ void store_y(YT* y, long long o, float v);
template <>
__device__ __forceinline__ void store_y<uint16_t>(uint16_t* y, long long o, float v) { y[o] = f32_to_bf16(v); }
template <>
__device__ __forceinline__ void store_y<float>(float* y, long long o, float v) { y[o] = v; }

template <typename YT>
__global__ __launch_bounds__(NTHR) void k_down_bf16(const uint16_t* __restrict__ h, const uint16_t* __restrict__ w2,
                                                    const int32_t* __restrict__ tile_map,
                                                    const int32_t* __restrict__ n_tiles, int d, int I,
                                                    YT* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][BM * LDA];
  const TileInfo ti = tile_of_block(tile_map, n_tiles, blockIdx.x);
  if (!ti.live) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.y * BN;  // first output column
  const uint16_t* wexp = w2 + (long long)ti.seg * d * I;

  const uint16_t* asrc[4];
  const uint16_t* bsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + NTHR * i;
    const int r = c >> 3, ch = c & 7;
    asrc[i] = r < ti.rows ? h + (long long)(ti.row0 + r) * I + ch * 8 : nullptr;
    bsrc[i] = wexp + (long long)(n0 + r) * I + ch * 8;
  }
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  Slab sa, sb;
  slab_load(sa, asrc, 0);
  slab_load(sb, bsrc, 0);
  slab_store(lds[0][0], sa, tid);
  slab_store(lds[0][1], sb, tid);
  __syncthreads();
  const int nk = I / BK;
  const int bn[2] = {wn * 64, wn * 64 + 32};
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      slab_load(sa, asrc, (kt + 1) * BK);
      slab_load(sb, bsrc, (kt + 1) * BK);
    }
    mma_slab(acc, lds[cur][0], lds[cur][1], wm * 64, bn, lane);
    if (kt + 1 < nk) {
      slab_store(lds[cur ^ 1][0], sa, tid);
      slab_store(lds[cur ^ 1][1], sb, tid);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = wm * 64 + i * 32 + acc_row(e, lane);
        if (r < ti.rows) {
          const int col = n0 + bn[j] + (lane & 31);
          store_y(y, (long long)(ti.row0 + r) * d + col, acc[i][j][e]);
        }
      }
}

// ------------------------------------------------------------ fp32 path --
// Plain LDS-tiled fp32 FMA kernels for fp32 layers (small shapes).  Tile:
// 64 rows x 64 columns x 16 K, 256 threads with 4 x 4 outputs each.
constexpr int FT = 64;
constexpr int FK = 16;

__device__ __forceinline__ void tile_of_block_f32(const int32_t* tile_map, const int32_t* n_tiles, int bx,
                                                  TileInfo& ti) {
  const int tile = bx >> 2, quarter = bx & 3;  // 256-row tiles in 64-row quarters
  ti.live = false;
  if (tile >= *n_tiles) return;
  const int4 m = *reinterpret_cast<const int4*>(tile_map + 4LL * tile);
  const int r = m.z - quarter * FT;
  if (r <= 0) return;
  ti.live = true;
  ti.seg = m.x;
  ti.row0 = m.y + quarter * FT;
  ti.rows = r < FT ? r : FT;
}

// out[r, n] = sum_k A[r, k] * W[n, k] for the block's 64 x 64 tile; A rows
// come from `arow` (nullptr = zero row).
__device__ __forceinline__ void f32_tile(const float* const* arow, const float* w, long long wstride, int n0, int ncols,
                                         int K, float (&acc)[4][4], float (*sa)[FT + 1], float (*sw)[FT + 1]) {
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;
  for (int k0 = 0; k0 < K; k0 += FK) {
    for (int i = tid; i < FT * FK; i += 256) {
      const int r = i / FK, c = i % FK;
      const int k = k0 + c;
      sa[c][r] = (arow[r] && k < K) ? arow[r][k] : 0.f;
      sw[c][r] = (r < ncols && k < K) ? w[(long long)(n0 + r) * wstride + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < FK; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(sa[c][tr * 4 + i], sw[c][tc * 4 + j], acc[i][j]);
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_gateup_f32(const float* __restrict__ x, const float* __restrict__ w13,
                                                    const int32_t* __restrict__ row_token,
                                                    const int32_t* __restrict__ tile_map,
                                                    const int32_t* __restrict__ n_tiles, int d, int I,
                                                    float* __restrict__ h) {
  __shared__ float sa[FK][FT + 1], sw[FK][FT + 1];
  __shared__ const float* arow[FT];
  TileInfo ti;
  tile_of_block_f32(tile_map, n_tiles, blockIdx.x, ti);
  if (!ti.live) return;
  const int c0 = blockIdx.y * FT;
  const int ncols = I - c0 < FT ? I - c0 : FT;
  const float* wexp = w13 + (long long)ti.seg * 2 * I * d;
  if (threadIdx.x < FT) {
    const int r = threadIdx.x;
    const int tok = r < ti.rows ? row_token[ti.row0 + r] : -1;
    arow[r] = tok >= 0 ? x + (long long)tok * d : nullptr;
  }
  __syncthreads();
  float g[4][4] = {}, up[4][4] = {};
  f32_tile(arow, wexp, d, c0, ncols, d, g, sa, sw);
  f32_tile(arow, wexp, d, I + c0, ncols, d, up, sa, sw);
  const int tr = threadIdx.x / 16, tc = threadIdx.x % 16;
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int r = tr * 4 + i, c = tc * 4 + j;
      if (r < ti.rows && c < ncols) h[(long long)(ti.row0 + r) * I + c0 + c] = silu(g[i][j]) * up[i][j];
    }
}

__global__ __launch_bounds__(256) void k_down_f32(const float* __restrict__ h, const float* __restrict__ w2,
                                                  const int32_t* __restrict__ tile_map,
                                                  const int32_t* __restrict__ n_tiles, int d, int I,
                                                  float* __restrict__ y) {
  __shared__ float sa[FK][FT + 1], sw[FK][FT + 1];
  __shared__ const float* arow[FT];
  TileInfo ti;
  tile_of_block_f32(tile_map, n_tiles, blockIdx.x, ti);
  if (!ti.live) return;
  const int n0 = blockIdx.y * FT;
  const int ncols = d - n0 < FT ? d - n0 : FT;
  if (threadIdx.x < FT) {
    const int r = threadIdx.x;
    arow[r] = r < ti.rows ? h + (long long)(ti.row0 + r) * I : nullptr;
  }
  __syncthreads();
  float acc[4][4] = {};
  f32_tile(arow, w2 + (long long)ti.seg * d * I, I, n0, ncols, I, acc, sa, sw);
  const int tr = threadIdx.x / 16, tc = threadIdx.x % 16;
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int r = tr * 4 + i, c = tc * 4 + j;
      if (r < ti.rows && c < ncols) y[(long long)(ti.row0 + r) * d + n0 + c] = acc[i][j];
    }
}

}  // namespace

void launch_ffn_bf16(const uint16_t* x, const uint16_t* w13, const uint16_t* w2, const int32_t* row_token,
                     const int32_t* tile_map, const int32_t* n_tiles, int tiles_max, int d, int I, uint16_t* h,
                     void* y, bool y_f32, hipStream_t st) {
  dim3 ga(tiles_max * 2, I / (BN / 2));
  hipLaunchKernelGGL(k_gateup_bf16, ga, dim3(NTHR), 0, st, x, w13, row_token, tile_map, n_tiles, d, I, h);
  dim3 gb(tiles_max * 2, d / BN);
  if (y_f32)
    hipLaunchKernelGGL(k_down_bf16<float>, gb, dim3(NTHR), 0, st, h, w2, tile_map, n_tiles, d, I,
                       static_cast<float*>(y));
  else
    hipLaunchKernelGGL(k_down_bf16<uint16_t>, gb, dim3(NTHR), 0, st, h, w2, tile_map, n_tiles, d, I,
                       static_cast<uint16_t*>(y));
}

void launch_ffn_f32(const float* x, const float* w13, const float* w2, const int32_t* row_token,
                    const int32_t* tile_map, const int32_t* n_tiles, int tiles_max, int d, int I, float* h, float* y,
                    hipStream_t st) {
  dim3 ga(tiles_max * 4, (unsigned)ceil_div(I, FT));
  hipLaunchKernelGGL(k_gateup_f32, ga, dim3(256), 0, st, x, w13, row_token, tile_map, n_tiles, d, I, h);
  dim3 gb(tiles_max * 4, (unsigned)ceil_div(d, FT));
  hipLaunchKernelGGL(k_down_f32, gb, dim3(256), 0, st, h, w2, tile_map, n_tiles, d, I, y);
}

}  // namespace moe
