// Bandwidth-bound steps of the layer: the gated combine, the bias rule and
// tile-wise E4M3 quantisation.
//
// Sources: "DeepSeek-V3 Technical Report" reading guide (xyznot.com), Method
// section 2 (combine equation, bias rule with gamma = 0.001) and "Key ideas",
// FP8 bullet (E4M3, 1x128 activation tiles, 128x128 weight blocks).
#include "common.h"

namespace moe {

namespace {

// ------------------------------------------------------------- combine --
// One block per token and 2048-column chunk; every thread owns 8 consecutive
// columns (16 B of bf16), so all loads are 16 B and coalesced.  The sum runs
// in fp32 in a fixed order: residual, shared experts, routed slots 0..K-1.
template <typename T_>
struct Vec8;
template <>
struct Vec8<uint16_t> {
  __device__ static void load(const uint16_t* p, float (&v)[8]) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static void store(uint16_t* p, const float (&v)[8]) {
    uint4 q;
    q.x = pack_bf16x2(v[0], v[1]);
    q.y = pack_bf16x2(v[2], v[3]);
    q.z = pack_bf16x2(v[4], v[5]);
    q.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = q;
  }
};
template <>
struct Vec8<float> {
  __device__ static void load(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ static void store(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// Raw 8-element vectors, kept as loaded until they are added (bf16 rows take
// 4 registers instead of 8).  Every byte is read once, so the loads are
// non-temporal (264 -> 231 us for the combine at T = 8192, d = 7168).
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  uint4 q;
  __device__ void load(const uint16_t* p) {
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
    q = make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ void get(float (&v)[8]) const {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct Raw8<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    const f32x4_nt x = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt*>(p));
    const f32x4_nt y = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt*>(p + 4));
    a = make_float4(x.x, x.y, x.z, x.w);
    b = make_float4(y.x, y.y, y.z, y.w);
  }
  __device__ void get(float (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

constexpr int CB_THREADS = 128;
constexpr int CB_COLS = CB_THREADS * 8;  // 1024 columns per block: d = 7168 is 7 blocks
constexpr int CB_SHARED = 2;              // shared rows gathered up front (more are added one by one)

// One block per (token, 1024 columns); a thread holds 8 columns.  The rows
// of the token are loaded before they are added, so their latencies
// overlap; the sum is formed in the fixed order u, shared rows, routed rows
// k = 0..K-1 (fp32, one rounding at the end), which keeps the result
// independent of the launch shape.
template <typename UT, typename YT, typename OT>
__global__ __launch_bounds__(CB_THREADS) void k_combine(const UT* __restrict__ u, const YT* __restrict__ y,
                                                        const int32_t* __restrict__ inv_row,
                                                        const float* __restrict__ gate,
                                                        const int32_t* __restrict__ seg_offset, int T, int d, int K,
                                                        int Nr, int Ns, unsigned flags, OT* __restrict__ out) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * CB_COLS + threadIdx.x * 8;
  if (c >= d) return;
  const bool res = !(flags & MOE_COMBINE_NO_RESIDUAL), sh = !(flags & MOE_COMBINE_NO_SHARED),
             ro = !(flags & MOE_COMBINE_NO_ROUTED);
  Raw8<UT> vu;
  Raw8<YT> vs[CB_SHARED], vr[MOE_MAX_K];
  float g[MOE_MAX_K];
  if (res) vu.load(u + (long long)t * d + c);
#pragma unroll
  for (int j = 0; j < CB_SHARED; ++j)
    if (sh && j < Ns) vs[j].load(y + ((long long)seg_offset[Nr + j] + t) * d + c);
#pragma unroll
  for (int k = 0; k < MOE_MAX_K; ++k)
    if (ro && k < K) {
      g[k] = gate[(long long)t * K + k];
      vr[k].load(y + (long long)inv_row[(long long)t * K + k] * d + c);
    }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0}, v[8];
  if (res) {
    vu.get(v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  if (sh) {
#pragma unroll
    for (int j = 0; j < CB_SHARED; ++j)
      if (j < Ns) {
        vs[j].get(v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
      }
    for (int j = CB_SHARED; j < Ns; ++j) {
      Vec8<YT>::load(y + ((long long)seg_offset[Nr + j] + t) * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
  }
#pragma unroll
  for (int k = 0; k < MOE_MAX_K; ++k)
    if (ro && k < K) {
      vr[k].get(v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[k], v[i], acc[i]);
    }
  Vec8<OT>::store(out + (long long)t * d + c, acc);
}

template <typename UT, typename YT, typename OT>
void launch_combine(const void* u, const void* y, const int32_t* inv_row, const float* gate, const int32_t* seg_offset,
                    int T, int d, int K, int Nr, int Ns, unsigned flags, void* out, hipStream_t st) {
  dim3 grid(T, (unsigned)ceil_div(d, CB_COLS));
  hipLaunchKernelGGL((k_combine<UT, YT, OT>), grid, dim3(CB_THREADS), 0, st, static_cast<const UT*>(u),
                     static_cast<const YT*>(y), inv_row, gate, seg_offset, T, d, K, Nr, Ns, flags,
                     static_cast<OT*>(out));
}

// ------------------------------------------------------ fused combine --
// Set-up of the fused combine (moe_expert_gemm_combine): out[t, :] = u[t, :]
// widened to fp32 (0 without the residual), and the gate of every token row
// of the layout: g[t, k] at row inv_row[t, k], 1 at the shared rows of t (0
// for a dropped term).  One block per token; padding rows are never read.
template <typename UT>
__global__ __launch_bounds__(256) void k_fused_prep(const UT* __restrict__ u, const int32_t* __restrict__ inv_row,
                                                    const float* __restrict__ gate,
                                                    const int32_t* __restrict__ seg_offset, int d, int K, int Nr,
                                                    int Ns, unsigned flags, float* __restrict__ out,
                                                    float* __restrict__ row_gate) {
  const int t = blockIdx.x, tid = threadIdx.x;
  const bool res = !(flags & MOE_COMBINE_NO_RESIDUAL), sh = !(flags & MOE_COMBINE_NO_SHARED),
             ro = !(flags & MOE_COMBINE_NO_ROUTED);
  for (int c = tid * 8; c < d; c += 256 * 8) {
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (res) Vec8<UT>::load(u + (long long)t * d + c, v);
    Vec8<float>::store(out + (long long)t * d + c, v);
  }
  for (int q = tid; q < K + Ns; q += 256) {
    if (q < K)
      row_gate[inv_row[(long long)t * K + q]] = ro ? gate[(long long)t * K + q] : 0.f;
    else
      row_gate[(long long)seg_offset[Nr + q - K] + t] = sh ? 1.f : 0.f;
  }
}

// ---------------------------------------------------------------- bias --
__global__ void k_bias_update(const int32_t* __restrict__ load, int Nr, long long total, float gamma,
                              float* __restrict__ bias) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Nr) return;
  const long long lhs = (long long)Nr * (long long)load[i];
  const float b = bias[i];
  if (lhs > total)
    bias[i] = b - gamma;
  else if (lhs < total)
    bias[i] = b + gamma;
}

// ------------------------------------------------------------ quantise --
template <typename XT>
__device__ __forceinline__ float ld(const XT* p, long long i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, long long i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, long long i) { return bf16_to_f32(p[i]); }

// x * 2^-k is exact (a power of two) and lies in [-448, 448] for every x of
// the tile, so each code is the round-to-nearest-even of x / scale.
// 1 x 128 tiles: 16 lanes per tile, 8 values per lane, 16 tiles per block.
// A 1 x 128 tile of a row-major [rows, cols] array with cols % 128 == 0 is
// the contiguous run x[128 t, 128 t + 128), t = row * cols / 128 + column
// block, which is also the index of its scale.
__device__ __forceinline__ void load8(const float* x, long long o, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(x + o);
  const float4 b = *reinterpret_cast<const float4*>(x + o + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* x, long long o, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(x + o);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <typename XT>
__global__ __launch_bounds__(256) void k_quant_1x128(const XT* __restrict__ x, long long ntiles,
                                                     uint8_t* __restrict__ q, float* __restrict__ scale) {
  const long long tile = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool live = tile < ntiles;  // every lane takes part in the shuffles
  const long long o = tile * 128 + sub * 8;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (live) load8(x, o, v);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));  // the tile's 16 lanes
  const int k = pow2_scale_exp(amax);
  const float inv = exp2_int(-k);
  if (live) {
    uint2 w;
    w.x = e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    w.y = e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    *reinterpret_cast<uint2*>(q + o) = w;
    if (sub == 0) scale[tile] = exp2_int(k);
  }
}

// 128 x 128 blocks: one block of 256 threads per tile, 64 values per thread.
template <typename XT>
__global__ __launch_bounds__(256) void k_quant_128x128(const XT* __restrict__ x, long long rows, long long cols,
                                                       uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[4];
  const long long tc = cols / 128;
  const long long tr = blockIdx.x / tc, tcol = blockIdx.x % tc;
  const int tid = threadIdx.x;
  const int col = (tid & 31) * 4;        // 32 threads x 4 columns
  const int row0 = tid >> 5;             // 8 row groups
  float m = 0.f;
  for (int rr = row0; rr < 128; rr += 8) {
    const long long o = (tr * 128 + rr) * cols + tcol * 128 + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(ld(x, o + i)));
  }
  m = wave_max_f32(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int k = pow2_scale_exp(amax);
  const float sc = exp2_int(k), inv = exp2_int(-k);
  for (int rr = row0; rr < 128; rr += 8) {
    const long long o = (tr * 128 + rr) * cols + tcol * 128 + col;
    *reinterpret_cast<uint32_t*>(q + o) =
        e4m3x4(ld(x, o) * inv, ld(x, o + 1) * inv, ld(x, o + 2) * inv, ld(x, o + 3) * inv);
  }
  if (tid == 0) scale[blockIdx.x] = sc;
}

// Codes x tile scale back to values: 8 consecutive codes of one row per
// thread (they share a scale: 128 % 8 == 0).  e4m3_to_f32(code) * 2^k is
// exact in fp32, and in bf16 too when 2^k >= 2^-124 (the smallest code step,
// 2^-9 * 2^k, is then a bf16 subnormal step or coarser).
__device__ __forceinline__ void store8v(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8v(uint16_t* p, const float (&v)[8]) {
  uint4 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]);
  w.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = w;
}

template <typename OT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ q, const float* __restrict__ scale,
                                                 long long rows, long long cols, int tile_rows,
                                                 OT* __restrict__ out) {
  const long long chunks = rows * (cols / 8);
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= chunks) return;
  const long long r = i / (cols / 8), c = (i % (cols / 8)) * 8;
  const float sc = scale[(r / tile_rows) * (cols / 128) + c / 128];
  const uint2 w = *reinterpret_cast<const uint2*>(q + r * cols + c);
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = e4m3_to_f32((w.x >> (8 * j)) & 0xFFu) * sc;
    v[4 + j] = e4m3_to_f32((w.y >> (8 * j)) & 0xFFu) * sc;
  }
  store8v(out + r * cols + c, v);
}

// ------------------------------------------------- runs along the rows --
// E4M3 along the token axis of the permuted layout, the K axis of the weight
// gradients: segment e (rows seg_offset[e] .. seg_offset[e + 1] - 1) is cut
// into runs of 128 rows from its first row, the last run shorter, and each
// column of a run gets its own power-of-two scale (the R10 rule).  Run r of
// segment e has scale row run_offset[e] + r.  Segment bounds are clamped to
// [0, P], so any seg_offset keeps every access inside the buffers.

__device__ __forceinline__ void seg_bounds(const int32_t* seg_offset, int e, long long P, int& s0, int& s1) {
  const int a = seg_offset[e], b = seg_offset[e + 1];
  s0 = a < 0 ? 0 : (a > P ? (int)P : a);
  s1 = b < s0 ? s0 : (b > P ? (int)P : b);
}

// run_offset[e] = sum over e' < e of ceil(len(e') / 128); run_offset[n] the
// total.  One block: every thread sums a contiguous chunk of segments, then
// an exclusive scan of the 1024 chunk sums in LDS.
__global__ __launch_bounds__(1024) void k_run_offsets(const int32_t* __restrict__ seg_offset, int n, long long P,
                                                      int32_t* __restrict__ run_offset) {
  __shared__ int part[1024];
  const int t = threadIdx.x, per = (n + 1023) / 1024;
  const int e0 = min(t * per, n), e1 = min(e0 + per, n);
  int sum = 0;
  for (int e = e0; e < e1; ++e) {
    int s0, s1;
    seg_bounds(seg_offset, e, P, s0, s1);
    sum += (s1 - s0 + 127) / 128;
  }
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - sum;
  for (int e = e0; e < e1; ++e) {
    run_offset[e] = run;
    int s0, s1;
    seg_bounds(seg_offset, e, P, s0, s1);
    run += (s1 - s0 + 127) / 128;
  }
  if (t == 1023) run_offset[n] = part[1023];
}

// One block per (run, 256-column chunk); thread (rg, cg) = (tid / 32,
// tid % 32) holds rows 16 rg .. 16 rg + 15 of the run and columns
// 8 cg .. 8 cg + 7 of the chunk.  The column maxima meet in LDS; codes are
// RNE(x / scale) as in the tile quantisers.  Source row of permuted row r:
// row_token[r] (GATHER, x [x_rows, cols]) or r itself (x [P, cols]); a row
// whose row_token is negative (padding), or names no row of x, counts as
// zeros, and its codes are written as 0.  ROW1 (x [P, cols]): the same
// values are also quantised in 1x128 row tiles into q_tile [P, cols] and
// s_tile [P, cols / 128], as k_quant_1x128 does, so a tensor that needs both
// layouts is read once; rows outside every segment are not written.
template <typename XT, bool GATHER, bool ROW1>
__global__ __launch_bounds__(256) void k_quant_runs(const XT* __restrict__ x, long long x_rows, int cols,
                                                    const int32_t* __restrict__ row_token,
                                                    const int32_t* __restrict__ seg_offset,
                                                    const int32_t* __restrict__ run_offset, int n, long long P,
                                                    uint8_t* __restrict__ q, float* __restrict__ scale,
                                                    uint8_t* __restrict__ q_tile, float* __restrict__ s_tile) {
  __shared__ float red[8][256];
  __shared__ int kexp[256];
  const int g = blockIdx.x;
  if (g >= run_offset[n]) return;
  int lo = 0, hi = n;  // run_offset[lo] <= g < run_offset[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (run_offset[mid] <= g) lo = mid; else hi = mid;
  }
  int s0, s1;
  seg_bounds(seg_offset, lo, P, s0, s1);
  const int row0 = s0 + 128 * (g - run_offset[lo]);
  const int row_end = min(row0 + 128, s1);
  const int tid = threadIdx.x, cg = tid & 31, rg = tid >> 5;
  const int c0 = blockIdx.y * 256, col = c0 + 8 * cg;
  const bool live_col = col < cols;
  // Every load is issued unconditionally (a row that has no source reads
  // a row that exists and is zeroed after), so the 16 row_token loads and
  // then the 16 data loads of a thread are in flight together; loads under
  // a per-row branch were issued and waited for one at a time.
  int tok[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = row0 + 16 * rg + r;
    tok[r] = row_token[row < row_end ? row : row_end - 1];
  }
  // a gathered x without rows is never read (it may be NULL)
  const bool readable = !GATHER || x_rows > 0;
  const int ccol = live_col ? col : 0;
  float v[16][8];
  if (readable) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = row0 + 16 * rg + r;
      const bool ok = live_col && row < row_end && tok[r] >= 0 && (!GATHER || tok[r] < x_rows);
      const long long src = ok ? (GATHER ? (long long)tok[r] : (long long)row) : (GATHER ? 0LL : (long long)row0);
      load8(x, src * cols + ccol, v[r]);
#pragma unroll
      for (int c = 0; c < 8; ++c) v[r][c] = ok ? v[r][c] : 0.f;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) v[r][c] = 0.f;
  }
  if constexpr (ROW1) {
    // a row's 1x128 tile is held by the 16 lanes of a wave with this rg and
    // this half of the 256-column chunk (lane bits 0-3 = cg & 15)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float m = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) m = fmaxf(m, fabsf(v[r][c]));
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
      const int k = pow2_scale_exp(m);
      const float iv = exp2_int(-k);
      const int row = row0 + 16 * rg + r;
      if (live_col && row < row_end) {
        uint2 w;
        w.x = e4m3x4(v[r][0] * iv, v[r][1] * iv, v[r][2] * iv, v[r][3] * iv);
        w.y = e4m3x4(v[r][4] * iv, v[r][5] * iv, v[r][6] * iv, v[r][7] * iv);
        *reinterpret_cast<uint2*>(q_tile + (long long)row * cols + col) = w;
        if ((cg & 15) == 0) s_tile[(long long)row * (cols / 128) + col / 128] = exp2_int(k);
      }
    }
  }
  float am[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 16; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) am[c] = fmaxf(am[c], fabsf(v[r][c]));
#pragma unroll
  for (int c = 0; c < 8; ++c) red[rg][8 * cg + c] = am[c];
  __syncthreads();
  {
    float m = red[0][tid];
#pragma unroll
    for (int r = 1; r < 8; ++r) m = fmaxf(m, red[r][tid]);
    const int k = pow2_scale_exp(m);
    kexp[tid] = k;
    if (c0 + tid < cols) scale[(long long)g * cols + c0 + tid] = exp2_int(k);
  }
  __syncthreads();
  if (!live_col) return;
  float inv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) inv[c] = exp2_int(-kexp[8 * cg + c]);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = row0 + 16 * rg + r;
    if (row < row_end) {
      uint2 w;
      w.x = e4m3x4(v[r][0] * inv[0], v[r][1] * inv[1], v[r][2] * inv[2], v[r][3] * inv[3]);
      w.y = e4m3x4(v[r][4] * inv[4], v[r][5] * inv[5], v[r][6] * inv[6], v[r][7] * inv[7]);
      *reinterpret_cast<uint2*>(q + (long long)row * cols + col) = w;
    }
  }
}

}  // namespace

moe_status combine(const void* u, moe_dtype u_t, const void* y, moe_dtype y_t, const int32_t* inv_row,
                   const float* topk_gate, const int32_t* seg_offset, int T, int d, int K, int Nr, int Ns,
                   unsigned flags, void* out, moe_dtype out_t, void* stream) {
  MOE_REQUIRE(T >= 0 && d >= 8 && d % 8 == 0, MOE_EINVAL, "need T >= 0 and d a positive multiple of 8");
  MOE_REQUIRE(Nr >= 1 && Ns >= 0 && Nr + Ns <= MOE_MAX_EXPERTS, MOE_EINVAL, "expert counts out of range");
  MOE_REQUIRE(K >= 1 && K <= MOE_MAX_K && K <= Nr, MOE_EINVAL, "K out of range");
  MOE_REQUIRE((flags & ~7u) == 0, MOE_EINVAL, "unknown flag bits");
  MOE_REQUIRE(u_t == MOE_F32 || u_t == MOE_BF16, MOE_EINVAL, "u_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(y_t == MOE_F32 || y_t == MOE_BF16, MOE_EINVAL, "y_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(out_t == MOE_F32 || out_t == MOE_BF16, MOE_EINVAL, "out_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(T == 0 || (u && y && inv_row && topk_gate && seg_offset && out), MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(out != y, MOE_EINVAL, "out aliases y");
  MOE_REQUIRE(aligned16(u) && aligned16(y) && aligned16(out), MOE_EINVAL, "u, y and out must be 16-byte aligned");
  if (T == 0) return MOE_OK;
  hipStream_t st = as_stream(stream);
  const int key = (u_t == MOE_BF16) * 4 + (y_t == MOE_BF16) * 2 + (out_t == MOE_BF16);
  using B = uint16_t;
  using F = float;
  switch (key) {
    case 0: launch_combine<F, F, F>(u, y, inv_row, topk_gate, seg_offset, T, d, K, Nr, Ns, flags, out, st); break;
    case 1: launch_combine<F, F, B>(u, y, inv_row, topk_gate, seg_offset, T, d, K, Nr, Ns, flags, out, st); break;
    case 2: launch_combine<F, B, F>(u, y, inv_row, topk_gate, seg_offset, T, d, K, Nr, Ns, flags, out, st); break;
    case 3: launch_combine<F, B, B>(u, y, inv_row, topk_gate, seg_offset, T, d, K, Nr, Ns, flags, out, st); break;
    case 4: launch_combine<B, F, F>(u, y, inv_row, topk_gate, seg_offset, T, d, K, Nr, Ns, flags, out, st); break;
    case 5: launch_combine<B, F, B>(u, y, inv_row, topk_gate, seg_offset, T, d, K, Nr, Ns, flags, out, st); break;
    case 6: launch_combine<B, B, F>(u, y, inv_row, topk_gate, seg_offset, T, d, K, Nr, Ns, flags, out, st); break;
    default: launch_combine<B, B, B>(u, y, inv_row, topk_gate, seg_offset, T, d, K, Nr, Ns, flags, out, st); break;
  }
  return launch_status("moe_combine");
}

moe_status bias_update(const int32_t* expert_load, int Nr, long long total_assign, float gamma, float* bias,
                       void* stream) {
  MOE_REQUIRE(expert_load && bias, MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(Nr >= 1 && Nr <= MOE_MAX_EXPERTS, MOE_EINVAL, "Nr out of range");
  MOE_REQUIRE(total_assign >= 0, MOE_EINVAL, "total_assign < 0");
  MOE_REQUIRE(std::isfinite(gamma) && gamma >= 0.f, MOE_EINVAL, "gamma must be finite and >= 0");
  hipLaunchKernelGGL(k_bias_update, dim3((Nr + 255) / 256), dim3(256), 0, as_stream(stream), expert_load, Nr,
                     total_assign, gamma, bias);
  return launch_status("moe_bias_update");
}

moe_status quantize_tiles(const void* x, moe_dtype x_t, long long rows, long long cols, int tile_rows, int tile_cols,
                          uint8_t* q, float* scale, void* stream) {
  MOE_REQUIRE(x_t == MOE_F32 || x_t == MOE_BF16, MOE_EINVAL, "x_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(tile_cols == 128 && (tile_rows == 1 || tile_rows == 128), MOE_EINVAL,
              "tiles must be 1x128 or 128x128");
  MOE_REQUIRE(rows >= 0 && cols >= 0 && cols % 128 == 0 && rows % tile_rows == 0, MOE_EINVAL,
              "rows/cols must be multiples of the tile");
  MOE_REQUIRE(rows == 0 || cols == 0 || (x && q && scale), MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(aligned16(x) && aligned16(q), MOE_EINVAL, "x and q must be 16-byte aligned");
  const long long ntiles = (rows / tile_rows) * (cols / 128);
  if (ntiles == 0) return MOE_OK;
  MOE_REQUIRE(ntiles < (1LL << 31) * 4, MOE_EINVAL, "too many tiles");
  hipStream_t st = as_stream(stream);
  if (tile_rows == 1) {
    dim3 grid((unsigned)ceil_div(ntiles, 16));
    if (x_t == MOE_F32)
      hipLaunchKernelGGL(k_quant_1x128<float>, grid, dim3(256), 0, st, static_cast<const float*>(x), ntiles, q, scale);
    else
      hipLaunchKernelGGL(k_quant_1x128<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(x), ntiles, q,
                         scale);
  } else {
    dim3 grid((unsigned)ntiles);
    if (x_t == MOE_F32)
      hipLaunchKernelGGL(k_quant_128x128<float>, grid, dim3(256), 0, st, static_cast<const float*>(x), rows, cols, q,
                         scale);
    else
      hipLaunchKernelGGL(k_quant_128x128<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(x), rows,
                         cols, q, scale);
  }
  return launch_status("fp8_quantize_tiles");
}

moe_status dequantize_tiles(const uint8_t* q, const float* scale, long long rows, long long cols, int tile_rows,
                            int tile_cols, void* out, moe_dtype out_t, void* stream) {
  MOE_REQUIRE(out_t == MOE_F32 || out_t == MOE_BF16, MOE_EINVAL, "out_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(tile_cols == 128 && (tile_rows == 1 || tile_rows == 128), MOE_EINVAL,
              "tiles must be 1x128 or 128x128");
  MOE_REQUIRE(rows >= 0 && cols >= 0 && cols % 128 == 0 && rows % tile_rows == 0, MOE_EINVAL,
              "rows/cols must be multiples of the tile");
  MOE_REQUIRE(rows == 0 || cols == 0 || (q && scale && out), MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(aligned16(q) && aligned16(out), MOE_EINVAL, "q and out must be 16-byte aligned");
  const long long chunks = rows * (cols / 8);
  if (chunks == 0) return MOE_OK;
  MOE_REQUIRE(chunks < (1LL << 31) * 256, MOE_EINVAL, "too many values");
  hipStream_t st = as_stream(stream);
  dim3 grid((unsigned)ceil_div(chunks, 256));
  if (out_t == MOE_F32)
    hipLaunchKernelGGL(k_dequant<float>, grid, dim3(256), 0, st, q, scale, rows, cols, tile_rows,
                       static_cast<float*>(out));
  else
    hipLaunchKernelGGL(k_dequant<uint16_t>, grid, dim3(256), 0, st, q, scale, rows, cols, tile_rows,
                       static_cast<uint16_t*>(out));
  return launch_status("fp8_dequantize_tiles");
}

long long quantize_runs_max(long long P, int n_seg) { return (P + 127LL * n_seg) / 128; }

void launch_quantize_runs(const void* x, bool x_f32, long long x_rows, int cols, const int32_t* row_token,
                          bool gather, const int32_t* seg_offset, int n_seg, long long P, int32_t* run_offset,
                          bool offsets, uint8_t* q, float* scale, hipStream_t st, uint8_t* q1, float* s1) {
  if (offsets) hipLaunchKernelGGL(k_run_offsets, dim3(1), dim3(1024), 0, st, seg_offset, n_seg, P, run_offset);
  const long long runs = quantize_runs_max(P, n_seg);
  if (runs == 0 || cols == 0) return;
  const dim3 grid((unsigned)runs, (unsigned)((cols + 255) / 256));
#define QR_LAUNCH(XT, G, R1)                                                                                        \
  hipLaunchKernelGGL((k_quant_runs<XT, G, R1>), grid, dim3(256), 0, st, static_cast<const XT*>(x), x_rows, cols,   \
                     row_token, seg_offset, run_offset, n_seg, P, q, scale, q1, s1)
  const bool row1 = q1 != nullptr && !gather;  // 1x128 tiles as well (x [P, cols])
  if (x_f32) {
    if (gather) QR_LAUNCH(float, true, false); else if (row1) QR_LAUNCH(float, false, true); else QR_LAUNCH(float, false, false);
  } else {
    if (gather) QR_LAUNCH(uint16_t, true, false); else if (row1) QR_LAUNCH(uint16_t, false, true); else QR_LAUNCH(uint16_t, false, false);
  }
#undef QR_LAUNCH
}

moe_status quantize_runs(const void* x, moe_dtype x_t, long long x_rows, int cols, const int32_t* row_token,
                         int gather, const int32_t* seg_offset, int n_seg, long long P, int32_t* run_offset,
                         uint8_t* q, float* scale, void* stream) {
  MOE_REQUIRE(x_t == MOE_F32 || x_t == MOE_BF16, MOE_EINVAL, "x_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(n_seg >= 1 && n_seg <= (1 << 20), MOE_EINVAL, "n_seg out of range");
  MOE_REQUIRE(P >= 0 && P < (1LL << 31) && cols >= 0 && cols % 128 == 0, MOE_EINVAL,
              "P must be in [0, 2^31) and cols a multiple of 128");
  MOE_REQUIRE(x_rows >= 0 && (gather || x_rows >= P), MOE_EINVAL, "x must have P rows unless gathered");
  MOE_REQUIRE(seg_offset && run_offset && row_token, MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(P == 0 || cols == 0 || (q && scale), MOE_EINVAL, "NULL pointer");
  // x is read only at rows that exist: none when a gathered x has no rows
  MOE_REQUIRE(x || cols == 0 || (gather ? x_rows == 0 : P == 0), MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(aligned16(x) && aligned16(q), MOE_EINVAL, "x and q must be 16-byte aligned");
  MOE_REQUIRE(fits31((unsigned long long)(gather ? x_rows : P) * cols * (x_t == MOE_F32 ? 4 : 2)) &&
                  fits31((unsigned long long)P * cols) &&
                  fits31((unsigned long long)quantize_runs_max(P, n_seg) * cols * 4),
              MOE_EUNSUPPORTED, "fp8_quantize_runs: operand of 2 GiB or more");
  launch_quantize_runs(x, x_t == MOE_F32, x_rows, cols, row_token, gather != 0, seg_offset, n_seg, P, run_offset,
                       true, q, scale, as_stream(stream), nullptr, nullptr);
  return launch_status("fp8_quantize_runs");
}

void launch_fused_combine_prep(const void* u, moe_dtype u_t, const int32_t* inv_row, const float* topk_gate,
                               const int32_t* seg_offset, int T, int d, int K, int Nr, int Ns, unsigned flags,
                               float* out, float* row_gate, hipStream_t st) {
  if (u_t == MOE_BF16)
    hipLaunchKernelGGL(k_fused_prep<uint16_t>, dim3(T), dim3(256), 0, st, static_cast<const uint16_t*>(u), inv_row,
                       topk_gate, seg_offset, d, K, Nr, Ns, flags, out, row_gate);
  else
    hipLaunchKernelGGL(k_fused_prep<float>, dim3(T), dim3(256), 0, st, static_cast<const float*>(u), inv_row,
                       topk_gate, seg_offset, d, K, Nr, Ns, flags, out, row_gate);
}

}  // namespace moe
