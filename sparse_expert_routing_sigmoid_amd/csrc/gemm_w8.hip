// Grouped SwiGLU expert GEMMs with E4M3 weights and bf16 activations, for
// few rows per expert (decode): a weight-streaming kernel.
//
// The expert FFNs of the combine equation in the "DeepSeek-V3 Technical
// Report" reading guide (xyznot.com, Method section 2), SwiGLU form, with the
// weights stored as in the same page's "Key ideas" FP8 bullet: E4M3 codes in
// 128x128 blocks, one power-of-two scale per block; the activations stay
// bf16.  With a handful of rows per expert the work is bound by streaming the
// weights from HBM once, so the kernel is built around that stream.
//
// Work item: (tile of the tile map, N tile).  Phase A: N tile = 128 h
// columns = 128 gate rows + the 128 up rows of the same columns of W13.
// Phase B: N tile = 256 columns of y (rows of W2).  A block is four waves;
// each wave owns four 16-row weight fragments (phase A: two gate + the two
// matching up fragments) over the whole K and keeps them out of LDS: weight
// bytes go global -> registers with 16-byte buffer loads, two K steps in
// flight, are widened to bf16 with the block scale folded in by the scaled
// E4M3 -> bf16 conversion (exact: the scale is a power of two), and feed
// 16x16x32 bf16 MFMAs with fp32 accumulators.  The rows of the tile are taken
// 16 * MC at a time (MC = 1 or 2); their activations come from L2.
// Scheduling barriers keep each step's loads together and in issue order,
// so the wait before a step's MFMAs covers only that step's loads.
//
// K order inside a step.  One K step covers 128 values (one scale block).
// Lane l holds column (or row) l % 16 and, with g = l / 16, the 16 K values
// [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16) of the step; each MFMA uses 8
// of them.  A and B use the same assignment, so every product pairs equal K
// indices and the sum over the step is the plain dot product whatever K order
// the hardware uses inside an MFMA.  A row of weights is read as two 64-byte
// runs per step, issued back to back.
#include "common.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_v __attribute__((ext_vector_type(4)));

constexpr int W8_THREADS = 256;  // four waves
constexpr int W8_NB = 4;         // 16-row weight fragments per wave
constexpr uint32_t W8_OOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t w8_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4_v ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}


// 16 E4M3 codes (one 16-byte load) times `scale` -> 2 x 8 bf16, K order kept.
__device__ __forceinline__ void widen16(u32x4_v q, float scale, bf16x8_v& lo, bf16x8_v& hi) {
  bf16x2_v p[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[2 * j] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[j], scale, false);
    p[2 * j + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[j], scale, true);
  }
  lo = bf16x8_v{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  hi = bf16x8_v{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
}

// Registers of one K step: per weight fragment two 16-byte runs; per 16-row
// group of activations four 16-byte runs.
template <int MC>
struct W8Step {
  u32x4_v b[W8_NB][2];
  u32x4_v a[MC][4];
};

struct W8Lanes {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t b_off[W8_NB];  // byte offset of this lane's weight row, K run 16g included
  int lane, g, c;
};

template <int MC>
__device__ __forceinline__ void w8_load(W8Step<MC>& st, const W8Lanes& L, const uint32_t (&a_off)[2], int k, int nk) {
  const uint32_t oob = k < nk ? 0u : W8_OOB;  // past the last step: zero loads that fetch nothing
  const uint32_t kb = (uint32_t)k * 128u;   // weight bytes (E4M3) before this step
#pragma unroll
  for (int f = 0; f < W8_NB; ++f) {
    st.b[f][0] = ld16(L.rb, L.b_off[f] | oob, kb);
    st.b[f][1] = ld16(L.rb, L.b_off[f] | oob, kb + 64u);
  }
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    const uint32_t ao = a_off[m] | oob;
    st.a[m][0] = ld16(L.ra, ao, 2u * kb);
    st.a[m][1] = ld16(L.ra, ao, 2u * kb + 16u);
    st.a[m][2] = ld16(L.ra, ao, 2u * kb + 128u);
    st.a[m][3] = ld16(L.ra, ao, 2u * kb + 144u);
  }
}

template <int MC>
__device__ __forceinline__ void w8_mma(f32x4_v (&acc)[MC][W8_NB], const W8Step<MC>& st, float s_lo, float s_hi) {
  // fragments 0, 1 use s_lo; 2, 3 use s_hi (phase A: gate / up block scales)
#pragma unroll
  for (int f = 0; f < W8_NB; ++f) {
    const float sc = f < 2 ? s_lo : s_hi;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8_v b0, b1;
      widen16(st.b[f][h], sc, b0, b1);
#pragma unroll
      for (int m = 0; m < MC; ++m) {
        acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, st.a[m][2 * h]), b0,
                                                            acc[m][f], 0, 0, 0);
        acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, st.a[m][2 * h + 1]), b1,
                                                            acc[m][f], 0, 0, 0);
      }
    }
  }
}

__device__ __forceinline__ void w8_store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
__device__ __forceinline__ void w8_store(float* p, float v) { *p = v; }

// One pass over the weights for rows [m0, m0 + 16 MC) of the tile.
// sc_lo / sc_hi: lane l holds the block scale of K block l of the wave's
// first / second fragment pair.
template <bool PHASE_A, int MC, typename OT>
__device__ __forceinline__ void w8_pass(const W8Lanes& L, const int32_t* __restrict__ row_token, int row0, int rows,
                                        int m0, int nk, uint32_t x_row_bytes, float sc_lo, float sc_hi,
                                        OT* __restrict__ out, long long out_ld, int col0) {
  uint32_t a_off[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int r = m0 + m * 16 + L.c;  // tile row of this lane in group m
    int src = -1;
    if (m < MC && r < rows) src = PHASE_A ? row_token[row0 + r] : row0 + r;
    a_off[m] = src >= 0 ? (uint32_t)src * x_row_bytes + (uint32_t)L.g * 32u : W8_OOB;
  }
  f32x4_v acc[MC][W8_NB];
#pragma unroll
  for (int m = 0; m < MC; ++m)
#pragma unroll
    for (int f = 0; f < W8_NB; ++f) acc[m][f] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  W8Step<MC> s0, s1;
  w8_load<MC>(s0, L, a_off, 0, nk);
  __builtin_amdgcn_sched_barrier(0);
  w8_load<MC>(s1, L, a_off, 1, nk);
  __builtin_amdgcn_sched_barrier(0);
  for (int k = 0; k < nk; k += 2) {  // nk is even
    const float lo0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_lo), k));
    const float hi0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_hi), k));
    w8_mma<MC>(acc, s0, lo0, hi0);
    __builtin_amdgcn_sched_barrier(0);
    w8_load<MC>(s0, L, a_off, k + 2, nk);
    __builtin_amdgcn_sched_barrier(0);
    const float lo1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_lo), k + 1));
    const float hi1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_hi), k + 1));
    w8_mma<MC>(acc, s1, lo1, hi1);
    __builtin_amdgcn_sched_barrier(0);
    w8_load<MC>(s1, L, a_off, k + 3, nk);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Accumulator element i of lane l: row 4 (l / 16) + i, column l % 16.
#pragma unroll
  for (int m = 0; m < MC; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m0 + m * 16 + 4 * L.g + i;
      if (r >= rows) continue;
      OT* orow = out + (long long)(row0 + r) * out_ld + col0 + L.c;
      if (PHASE_A) {
#pragma unroll
        for (int f = 0; f < 2; ++f) w8_store(orow + f * 16, silu(acc[m][f][i]) * acc[m][f + 2][i]);
      } else {
#pragma unroll
        for (int f = 0; f < W8_NB; ++f) w8_store(orow + f * 16, acc[m][f][i]);
      }
    }
}

// PHASE_A: x = tokens [T, Kd] bf16 gathered by row_token, w = W13 codes
//          [E, 2 Nd, Kd], out = h [P, Nd] bf16 with SwiGLU; Nd = I, Kd = d.
// !PHASE_A: x = h [P, Kd] bf16, w = W2 codes [E, Nd, Kd], out = y [P, Nd].
// w_scale: [E, rows of w / 128, Kd / 128] powers of two.
// The items of one launch part are run by `nblocks` blocks; this block is
// number `block` of them.
template <bool PHASE_A, typename OT>
__device__ __forceinline__ void w8_items(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
                                         const float* __restrict__ w_scale, const int32_t* __restrict__ row_token,
                                         const int32_t* __restrict__ tile_map, const int32_t* __restrict__ n_tiles,
                                         int Kd, int Nd, uint32_t x_bytes, int part, int parts,
                                         OT* __restrict__ out, int block, int nblocks) {
  constexpr int NCOL = PHASE_A ? 128 : 256;  // output columns per item
  const int NT = Nd / NCOL;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nk = Kd / 128;  // K steps = K blocks
  const int wrows = PHASE_A ? 2 * Nd : Nd;
  const long long w_expert = (long long)wrows * Kd;
  // this launch covers tiles [t_lo, t_hi) of the tile map (part of parts)
  const int all_tiles = *n_tiles;
  const int t_lo = (int)((long long)all_tiles * part / parts), t_hi = (int)((long long)all_tiles * (part + 1) / parts);
  const int tiles = t_hi - t_lo;
  const long long total = (long long)tiles * NT;
  for (long long item = block; item < total; item += nblocks) {
    // shared-expert tiles (at the end of the tile map, the largest) go first
    const int tile = t_hi - 1 - (int)(item / NT);
    const int n = (int)(item % NT);
    const int4 tm = *reinterpret_cast<const int4*>(tile_map + 4LL * tile);
    const int seg = tm.x, row0 = tm.y, rows = tm.w;  // token rows only

    W8Lanes L;
    L.lane = lane;
    L.g = lane >> 4;
    L.c = lane & 15;
    L.ra = w8_rsrc(x, x_bytes);
    L.rb = w8_rsrc(w + seg * w_expert, (uint32_t)w_expert);
    int blk_lo, blk_hi;  // 128-row scale blocks of the fragment pairs
#pragma unroll
    for (int f = 0; f < W8_NB; ++f) {
      int wrow;
      if (PHASE_A)
        wrow = (f < 2 ? 0 : Nd) + n * 128 + wave * 32 + (f & 1) * 16;  // gate, gate, up, up
      else
        wrow = n * 256 + wave * 64 + f * 16;
      L.b_off[f] = (uint32_t)(wrow + L.c) * (uint32_t)Kd + (uint32_t)L.g * 16u;
    }
    if (PHASE_A) {
      blk_lo = n;
      blk_hi = Nd / 128 + n;
    } else {
      blk_lo = blk_hi = 2 * n + (wave >> 1);
    }
    const float* ws = w_scale + (long long)seg * (wrows / 128) * nk;
    const float sc_lo = lane < nk ? ws[(long long)blk_lo * nk + lane] : 1.0f;
    const float sc_hi = lane < nk ? ws[(long long)blk_hi * nk + lane] : 1.0f;
    const int col0 = PHASE_A ? n * 128 + wave * 32 : n * 256 + wave * 64;
    const uint32_t x_row_bytes = (uint32_t)Kd * 2u;
    for (int m0 = 0; m0 < rows;) {
      if (rows - m0 > 16) {
        w8_pass<PHASE_A, 2, OT>(L, row_token, row0, rows, m0, nk, x_row_bytes, sc_lo, sc_hi, out, Nd, col0);
        m0 += 32;
      } else {
        w8_pass<PHASE_A, 1, OT>(L, row_token, row0, rows, m0, nk, x_row_bytes, sc_lo, sc_hi, out, Nd, col0);
        m0 += 16;
      }
    }
  }
}

template <bool PHASE_A, typename OT>
__global__ __launch_bounds__(W8_THREADS) void k_ffn_w8a16(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
                                                          const float* __restrict__ w_scale,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ tile_map,
                                                          const int32_t* __restrict__ n_tiles, int Kd, int Nd,
                                                          uint32_t x_bytes, int part, int parts,
                                                          OT* __restrict__ out) {
  w8_items<PHASE_A, OT>(x, w, w_scale, row_token, tile_map, n_tiles, Kd, Nd, x_bytes, part, parts, out, blockIdx.x,
                        gridDim.x);
}

int w8_grid(long long items) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const long long cap = (long long)cus * 8;  // enough blocks for several resident waves per SIMD
  return (int)(items < cap ? (items > 0 ? items : 1) : cap);
}

}  // namespace

bool ffn_w8a16_ok(int d, int I) { return d % 256 == 0 && I % 256 == 0 && d / 128 <= 64 && I / 128 <= 64; }

// x [T, d] bf16; W13 / W2 E4M3 codes with 128x128 block scales; h (workspace)
// [P, I] bf16; y [P, d] bf16 or fp32.  tiles_max bounds the tile map.
//
// Four launches on the caller's stream: gate/up of tile halves 0 and 1, then
// down of halves 0 and 1.  Each half's grid is sized for its own items, so
// the tail of one launch (its last blocks, when most CUs are idle) is
// shorter than one launch over all tiles would leave.  Measured on the
// 128-token decode step: 1.90 ms per call, the same as running the down
// projection of half 0 on a second stream beside the gate/up of half 1
// (1.91-1.92 ms), and 2.09 ms when those two run as the two roles of one
// grid.
void launch_ffn_w8a16(const uint16_t* x, const uint8_t* w13, const float* w13_scale, const uint8_t* w2,
                      const float* w2_scale, const int32_t* row_token, const int32_t* tile_map,
                      const int32_t* n_tiles, int tiles_max, int T, long long P, int d, int I, uint16_t* h, void* y,
                      bool y_f32, hipStream_t st) {
  const uint32_t x_bytes = (uint32_t)((long long)T * d * 2);
  const uint32_t h_bytes = (uint32_t)(P * I * 2);
  const int half = (tiles_max + 1) / 2;
  const int gA = w8_grid((long long)half * (I / 128)), gB = w8_grid((long long)half * (d / 256));
  for (int part = 0; part < 2; ++part)
    hipLaunchKernelGGL((k_ffn_w8a16<true, uint16_t>), dim3(gA), dim3(W8_THREADS), 0, st, x, w13, w13_scale,
                       row_token, tile_map, n_tiles, d, I, x_bytes, part, 2, h);
  for (int part = 0; part < 2; ++part) {
    if (y_f32)
      hipLaunchKernelGGL((k_ffn_w8a16<false, float>), dim3(gB), dim3(W8_THREADS), 0, st, h, w2, w2_scale, row_token,
                         tile_map, n_tiles, I, d, h_bytes, part, 2, static_cast<float*>(y));
    else
      hipLaunchKernelGGL((k_ffn_w8a16<false, uint16_t>), dim3(gB), dim3(W8_THREADS), 0, st, h, w2, w2_scale,
                         row_token, tile_map, n_tiles, I, d, h_bytes, part, 2, static_cast<uint16_t*>(y));
  }
}

}  // namespace moe
