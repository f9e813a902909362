// Backward pass of the layer (bf16 path): the training forward that keeps
// the activations the backward needs, the gradient of the combine and of
// the gates, the expert GEMM gradients (gemm_bwd.hip) and the input and
// centroid gradients.
//
// The pages print no backward pass; every step is the chain rule through the
// forward of the "DeepSeek-V3 Technical Report" reading guide (xyznot.com),
// Method section 2: the combine equation, the affinity sentence (s =
// Sigmoid(u . e)) and the gate equation (g = s / sum of the selected s).
// The top-K selection and the bias only decide which gates exist: they are
// piecewise constant, so no gradient flows through them and the bias gets
// none.  With G = dL/dh':
//   dy[row(t, k)] = g_{t,k} G_t,   dy[shared row(t)] = G_t
//   dg_{t,k} = <G_t, y[row(t, k)]>
//   ds_{t,k} = (dg_{t,k} - sum_j g_{t,j} dg_{t,j}) / S_t,   S_t = sum_j s_{t,j}
//   dz_{t,k} = ds_{t,k} s_{t,k} (1 - s_{t,k})               (z = u . e)
//   du_t = G_t + sum of dx over the token's rows + sum_k dz_{t,k} e_{idx(t,k)}
//   de_i = sum over the rows of segment i of dz . u_t (the rows of segment i
//          are the tokens that selected expert i, each once)
#include "common.h"

namespace moe {

size_t permute_rows(int T, int K, int Nr, int Ns, int tile_m);
size_t permute_tiles_max(int T, int K, int Nr, int Ns, int tile_m);
size_t gemm_sched_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m);
bool ffn_bf16_persistent_ok(int d, int I);
int ffn_schedule_max_tiles();
void launch_ffn_bf16_persistent(const uint16_t* x, const uint16_t* w13, const uint16_t* w2, const int32_t* row_token,
                                const int32_t* tile_map, const int32_t* n_tiles, int T, long long P, int d, int I,
                                int Nr, int cap, uint16_t* h, uint16_t* ab, void* y, bool y_f32, int* sched,
                                hipStream_t st, const float* row_gate = nullptr);
bool ffn_bwd_ok(int d, int I);
bool ffn_bwd_w8_ok(int d, int I);
bool ffn_fp8_persistent_ok(int d, int I);
void launch_ffn_fp8_persistent(const uint8_t* x, const float* x_scale, const uint8_t* w13, const float* w13_scale,
                               const uint8_t* w2, const float* w2_scale, const int32_t* row_token,
                               const int32_t* tile_map, const int32_t* n_tiles, int T, long long P, int d, int I,
                               int Nr, int cap, uint8_t* h, float* h_scale, void* y, bool y_f32, int* sched,
                               hipStream_t st, uint16_t* ab, uint16_t* hb, const float* row_gate = nullptr);
void launch_ffn_bwd_w8(const uint16_t* x, const uint8_t* w13, const float* w13s, const uint8_t* w2, const float* w2s,
                       const uint16_t* h, const uint16_t* ab, const uint16_t* dy, const int32_t* seg_offset,
                       const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles, int tiles_max,
                       int T, long long P, int d, int I, int Nr, int Ns, uint16_t* dab, uint8_t* dyq, float* dys,
                       uint8_t* dabq, float* dabs, int* deal, uint16_t* dx, void* dw13, void* dw2, bool dw_f32,
                       hipStream_t st);
void launch_ffn_bwd_f8(const uint16_t* x, const uint8_t* w13, const float* w13s, const uint8_t* w2, const float* w2s,
                       const uint16_t* h, const uint16_t* ab, const uint16_t* dy, const int32_t* seg_offset,
                       const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles, int tiles_max,
                       int T, long long P, int d, int I, int Nr, int Ns, uint16_t* dab, uint8_t* dyq, float* dys,
                       uint8_t* dabq, float* dabs, uint8_t* hr, uint8_t* xr, uint8_t* dyr, uint8_t* dabr,
                       float* dyrs, float* hrs, float* dabrs, float* xrs, int32_t* run_offset, int* deal, uint16_t* dx,
                       void* dw13, void* dw2, bool dw_f32,
                       hipStream_t st);
long long quantize_runs_max(long long P, int n_seg);
void launch_ffn_bwd_bf16(const uint16_t* x, const uint16_t* w13, const uint16_t* w2, const uint16_t* h,
                         const uint16_t* ab, const uint16_t* dy, const int32_t* seg_offset, const int32_t* row_token,
                         const int32_t* tile_map, const int32_t* n_tiles, int tiles_max, int T, long long P, int d,
                         int I, int Nr, int Ns, uint16_t* dab, int* deal, uint16_t* dx, void* dw13, void* dw2,
                         bool dw_f32, hipStream_t st);

namespace {

// 8 consecutive values as fp32 (bf16 or fp32 storage), and back.
__device__ __forceinline__ void ld8(const uint16_t* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
// The same with the non-temporal hint, for rows read once (G, y, dx):
// 426 -> 410 us for the combine backward at T = 8192.  The centroid
// gradient re-reads token rows once per selected expert and keeps ld8.
__device__ __forceinline__ void ld8_once(const uint16_t* p, float (&v)[8]) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(q[i] << 16);
    v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void ld8_once(const float* p, float (&v)[8]) { ld8(p, v); }
__device__ __forceinline__ void st8(uint16_t* p, const float (&v)[8]) {
  uint4 q;
  q.x = pack_bf16x2(v[0], v[1]);
  q.y = pack_bf16x2(v[2], v[3]);
  q.z = pack_bf16x2(v[4], v[5]);
  q.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = q;
}
__device__ __forceinline__ void st8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <typename T>
const T* cp(const void* p) { return static_cast<const T*>(p); }

// ------------------------------------------------------- combine backward --
// One block per token.  Each thread owns 8 columns per pass over the row;
// the K dot products <G, y_k> are summed per thread in column order, then
// across the wave by a butterfly and across the 4 waves in wave order, so
// the result is the same on every run.
constexpr int CBB_THREADS = 256;

template <typename GT, typename YT>
__global__ __launch_bounds__(CBB_THREADS) void k_combine_bwd(const GT* __restrict__ G, const YT* __restrict__ y,
                                                             const int32_t* __restrict__ inv_row,
                                                             const float* __restrict__ gate,
                                                             const float* __restrict__ score,
                                                             const int32_t* __restrict__ seg_offset, int d, int K,
                                                             int Nr, int Ns, uint16_t* __restrict__ dy,
                                                             float* __restrict__ dgate, float* __restrict__ dz,
                                                             float* __restrict__ dz_row) {
  __shared__ float s_part[CBB_THREADS / 64][MOE_MAX_K];
  const int t = blockIdx.x, tid = threadIdx.x;
  long long rows[MOE_MAX_K];
  float g[MOE_MAX_K], part[MOE_MAX_K];
#pragma unroll
  for (int k = 0; k < MOE_MAX_K; ++k) {
    rows[k] = k < K ? inv_row[(long long)t * K + k] : 0;
    g[k] = k < K ? gate[(long long)t * K + k] : 0.f;
    part[k] = 0.f;
  }
  for (int c = tid * 8; c < d; c += CBB_THREADS * 8) {
    float gv[8], yv[8], o[8];
    ld8_once(G + (long long)t * d + c, gv);
#pragma unroll
    for (int k = 0; k < MOE_MAX_K; ++k) {
      if (k >= K) break;
      ld8_once(y + rows[k] * d + c, yv);
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) p = fmaf(gv[i], yv[i], p);
      part[k] += p;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = g[k] * gv[i];
      st8(dy + rows[k] * d + c, o);
    }
    for (int j = 0; j < Ns; ++j) st8(dy + ((long long)seg_offset[Nr + j] + t) * d + c, gv);
  }
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int k = 0; k < MOE_MAX_K; ++k) {
    if (k >= K) break;
    float v = part[k];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) s_part[wave][k] = v;
  }
  __syncthreads();
  if (tid == 0) {
    float dg[MOE_MAX_K], S = 0.f, gd = 0.f;
    for (int k = 0; k < K; ++k) {
      float v = 0.f;
      for (int w = 0; w < CBB_THREADS / 64; ++w) v += s_part[w][k];
      dg[k] = v;
      S += score[(long long)t * K + k];
      gd = fmaf(g[k], v, gd);
    }
    for (int k = 0; k < K; ++k) {
      const float s = score[(long long)t * K + k];
      const float z = (dg[k] - gd) / S * s * (1.0f - s);
      dgate[(long long)t * K + k] = dg[k];
      dz[(long long)t * K + k] = z;
      dz_row[rows[k]] = z;
    }
  }
}

// --------------------------------------------------------- input gradient --
// du_t = G_t + sum_j dx[shared row] + sum_k dx[row(t, k)] + sum_k dz_{t,k} e_{idx(t,k)},
// fp32, in that order; a block per (token, 1024 columns), 8 columns a thread.
constexpr int IG_THREADS = 128;
constexpr int IG_COLS = IG_THREADS * 8;

template <typename GT, typename OT>
__global__ __launch_bounds__(IG_THREADS) void k_input_grad(const GT* __restrict__ G, const uint16_t* __restrict__ dx,
                                                           const float* __restrict__ e,
                                                           const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ inv_row,
                                                           const float* __restrict__ dz,
                                                           const int32_t* __restrict__ seg_offset, int d, int K,
                                                           int Nr, int Ns, OT* __restrict__ du) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * IG_COLS + threadIdx.x * 8;
  if (c >= d) return;
  float acc[8], v[8];
  ld8_once(G + (long long)t * d + c, acc);
  for (int j = 0; j < Ns; ++j) {
    ld8_once(dx + ((long long)seg_offset[Nr + j] + t) * d + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  for (int k = 0; k < K; ++k) {
    ld8_once(dx + (long long)inv_row[(long long)t * K + k] * d + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  for (int k = 0; k < K; ++k) {
    const float z = dz[(long long)t * K + k];
    ld8(e + (long long)idx[(long long)t * K + k] * d + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(z, v[i], acc[i]);
  }
  st8(du + (long long)t * d + c, acc);
}

// ------------------------------------------------------ centroid gradient --
// de_i = sum over the token rows r of segment i of dz_row[r] u[row_token[r]].
// A block per (expert, 512 columns): 4 waves over the same columns, wave w
// taking rows w, w + 4, ... of the segment, eight rows at a time with the
// next eight tokens fetched ahead; the 4 partial sums are added in wave
// order, so the result is the same on every run.
constexpr int CG_THREADS = 256;
constexpr int CG_COLS = 512;

template <typename UT>
__global__ __launch_bounds__(CG_THREADS) void k_centroid_grad(const UT* __restrict__ u,
                                                              const int32_t* __restrict__ seg_offset,
                                                              const int32_t* __restrict__ row_token,
                                                              const float* __restrict__ dz_row, int d,
                                                              float* __restrict__ de) {
  __shared__ float4 s_part[3][64][2];
  const int i = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.y * CG_COLS + lane * 8;
  const bool col_ok = c < d;
  const int r0 = seg_offset[i], r1 = seg_offset[i + 1];
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, v[8];
  int tok[8];
  float z[8];
  auto fetch = [&](int base) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = base + 4 * q;
      tok[q] = r < r1 ? row_token[r] : -1;
      z[q] = r < r1 ? dz_row[r] : 0.f;
    }
  };
  fetch(r0 + wave);
  for (int base = r0 + wave; base < r1; base += 32) {
    int tk[8];
    float zz[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      tk[q] = tok[q];
      zz[q] = z[q];
    }
    fetch(base + 32);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (tk[q] < 0 || !col_ok) continue;
      ld8(u + (long long)tk[q] * d + c, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(zz[q], v[k], acc[k]);
    }
  }
  if (wave > 0) {
    s_part[wave - 1][lane][0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    s_part[wave - 1][lane][1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  __syncthreads();
  if (wave == 0 && col_ok) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      const float4 p = s_part[w][lane][0], q = s_part[w][lane][1];
      acc[0] += p.x; acc[1] += p.y; acc[2] += p.z; acc[3] += p.w;
      acc[4] += q.x; acc[5] += q.y; acc[6] += q.z; acc[7] += q.w;
    }
    st8(de + (long long)i * d + c, acc);
  }
}

}  // namespace

// ---------------------------------------------------------------- host --
size_t gemm_train_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  if (T < 0 || d < 1 || I < 1 || Nr < 1 || Ns < 0 || K < 1 || tile_m < 1) return 0;
  return gemm_sched_bytes(T, K, Nr, Ns, d, I, tile_m);
}

static moe_status check_layer(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  MOE_REQUIRE(T >= 0 && d >= 1 && I >= 1, MOE_EINVAL, "need T >= 0, d >= 1, I >= 1");
  MOE_REQUIRE(Nr >= 1 && Ns >= 0 && Nr + Ns <= MOE_MAX_EXPERTS, MOE_EINVAL, "expert counts out of range");
  MOE_REQUIRE(K >= 1 && K <= MOE_MAX_K && K <= Nr, MOE_EINVAL, "K out of range");
  MOE_REQUIRE(tile_m >= 1 && tile_m <= MOE_TILE_ROWS && (tile_m & (tile_m - 1)) == 0, MOE_EINVAL, "bad tile_m");
  return MOE_OK;
}

moe_status expert_gemm_train(const void* x, const void* w13, const void* w2, int T, int K, int Nr, int Ns, int d,
                             int I, int tile_m, const int32_t* seg_offset, const int32_t* row_token,
                             const int32_t* tile_map, const int32_t* n_tiles, void* ws, size_t ws_bytes, void* h,
                             void* ab, void* y, moe_dtype y_t, void* stream) {
  const moe_status cs = check_layer(T, K, Nr, Ns, d, I, tile_m);
  if (cs != MOE_OK) return cs;
  MOE_REQUIRE(y_t == MOE_F32 || y_t == MOE_BF16, MOE_EINVAL, "bad y_t");
  MOE_REQUIRE(w13 && w2 && seg_offset && row_token && tile_map && n_tiles && y && h && ab, MOE_EINVAL,
              "NULL pointer");
  MOE_REQUIRE(T == 0 || x, MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(aligned16(x) && aligned16(w13) && aligned16(w2) && aligned16(y) && aligned16(ws) && aligned16(h) &&
                  aligned16(ab),
              MOE_EINVAL, "x, w13, w2, h, ab, y and ws must be 16-byte aligned");
  MOE_REQUIRE(ffn_bf16_persistent_ok(d, I) && ffn_bwd_ok(d, I), MOE_EUNSUPPORTED,
              "training path needs d % 256 == 0, I % 128 == 0, d <= 65280, I <= 32640");
  const size_t P = permute_rows(T, K, Nr, Ns, tile_m);
  const int tiles_max = (int)permute_tiles_max(T, K, Nr, Ns, tile_m);
  MOE_REQUIRE(tiles_max <= ffn_schedule_max_tiles(), MOE_EUNSUPPORTED, "more GEMM tiles than the schedule holds");
  MOE_REQUIRE(fits31((unsigned long long)T * d * 2) && fits31((unsigned long long)P * d * 2) &&
                  fits31((unsigned long long)P * 2 * I * 2) && fits31((unsigned long long)3 * I * d * 2),
              MOE_EUNSUPPORTED, "training path: operand of 2 GiB or more");
  MOE_REQUIRE(ws && ws_bytes >= gemm_train_workspace_bytes(T, K, Nr, Ns, d, I, tile_m), MOE_EWORKSPACE,
              "workspace smaller than moe_gemm_train_workspace_bytes");
  if (T == 0) return MOE_OK;
  launch_ffn_bf16_persistent(cp<uint16_t>(x), cp<uint16_t>(w13), cp<uint16_t>(w2), row_token, tile_map, n_tiles, T,
                             (long long)P, d, I, Nr, tiles_max, static_cast<uint16_t*>(h),
                             static_cast<uint16_t*>(ab), y, y_t == MOE_F32, static_cast<int*>(ws),
                             as_stream(stream));
  return launch_status("moe_expert_gemm_train");
}

// Workspace of the E4M3 training forward: the work schedule, then h as E4M3
// codes [P, I] and its 1x128 scales [P, I / 128].
static size_t train_w8_h_offset(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  return (gemm_sched_bytes(T, K, Nr, Ns, d, I, tile_m) + 255) / 256 * 256;
}

size_t gemm_train_w8_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  if (T < 0 || d < 1 || I < 128 || Nr < 1 || Ns < 0 || K < 1 || tile_m < 1) return 0;
  const size_t P = permute_rows(T, K, Nr, Ns, tile_m);
  return train_w8_h_offset(T, K, Nr, Ns, d, I, tile_m) + (P * I + 255) / 256 * 256 + P * (size_t)(I / 128) * 4;
}

moe_status expert_gemm_train_w8(const uint8_t* x, const float* x_scale, const uint8_t* w13, const float* w13_scale,
                                const uint8_t* w2, const float* w2_scale, int T, int K, int Nr, int Ns, int d, int I,
                                int tile_m, const int32_t* seg_offset, const int32_t* row_token,
                                const int32_t* tile_map, const int32_t* n_tiles, void* ws, size_t ws_bytes, void* h,
                                void* ab, void* y, moe_dtype y_t, void* stream) {
  const moe_status cs = check_layer(T, K, Nr, Ns, d, I, tile_m);
  if (cs != MOE_OK) return cs;
  MOE_REQUIRE(y_t == MOE_F32 || y_t == MOE_BF16, MOE_EINVAL, "bad y_t");
  MOE_REQUIRE(w13 && w13_scale && w2 && w2_scale && seg_offset && row_token && tile_map && n_tiles && y && h && ab,
              MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(T == 0 || (x && x_scale), MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(aligned16(x) && aligned16(w13) && aligned16(w2) && aligned16(y) && aligned16(ws) && aligned16(h) &&
                  aligned16(ab),
              MOE_EINVAL, "x, w13, w2, h, ab, y and ws must be 16-byte aligned");
  MOE_REQUIRE(ffn_fp8_persistent_ok(d, I) && ffn_bwd_w8_ok(d, I), MOE_EUNSUPPORTED,
              "E4M3 training path needs d % 256 == 0, I % 256 == 0, d <= 8192, I <= 8192");
  const size_t P = permute_rows(T, K, Nr, Ns, tile_m);
  const int tiles_max = (int)permute_tiles_max(T, K, Nr, Ns, tile_m);
  MOE_REQUIRE(tiles_max <= ffn_schedule_max_tiles(), MOE_EUNSUPPORTED, "more GEMM tiles than the schedule holds");
  MOE_REQUIRE(fits31((unsigned long long)P * d * 2) && fits31((unsigned long long)P * 2 * I * 2) &&
                  fits31((unsigned long long)2 * I * d),
              MOE_EUNSUPPORTED, "training path: operand of 2 GiB or more");
  MOE_REQUIRE(ws && ws_bytes >= gemm_train_w8_workspace_bytes(T, K, Nr, Ns, d, I, tile_m), MOE_EWORKSPACE,
              "workspace smaller than moe_gemm_train_w8_workspace_bytes");
  if (T == 0) return MOE_OK;
  uint8_t* wb = static_cast<uint8_t*>(ws);
  const size_t ho = train_w8_h_offset(T, K, Nr, Ns, d, I, tile_m);
  uint8_t* hq = wb + ho;
  float* hs = reinterpret_cast<float*>(wb + ho + (P * I + 255) / 256 * 256);
  launch_ffn_fp8_persistent(x, x_scale, w13, w13_scale, w2, w2_scale, row_token, tile_map, n_tiles, T, (long long)P,
                            d, I, Nr, tiles_max, hq, hs, y, y_t == MOE_F32, reinterpret_cast<int*>(wb),
                            as_stream(stream), static_cast<uint16_t*>(ab), static_cast<uint16_t*>(h));
  return launch_status("moe_expert_gemm_train_w8");
}

moe_status combine_backward(const void* grad_out, moe_dtype g_t, const void* y, moe_dtype y_t,
                            const int32_t* inv_row, const float* topk_gate, const float* topk_score,
                            const int32_t* seg_offset, int T, int d, int K, int Nr, int Ns, void* dy, float* dgate,
                            float* dz, float* dz_row, void* stream) {
  MOE_REQUIRE(T >= 0 && d >= 8 && d % 8 == 0, MOE_EINVAL, "need T >= 0 and d a positive multiple of 8");
  MOE_REQUIRE(Nr >= 1 && Ns >= 0 && Nr + Ns <= MOE_MAX_EXPERTS, MOE_EINVAL, "expert counts out of range");
  MOE_REQUIRE(K >= 1 && K <= MOE_MAX_K && K <= Nr, MOE_EINVAL, "K out of range");
  MOE_REQUIRE(g_t == MOE_F32 || g_t == MOE_BF16, MOE_EINVAL, "g_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(y_t == MOE_F32 || y_t == MOE_BF16, MOE_EINVAL, "y_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(T == 0 || (grad_out && y && inv_row && topk_gate && topk_score && seg_offset && dy && dgate && dz &&
                         dz_row),
              MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(aligned16(grad_out) && aligned16(y) && aligned16(dy), MOE_EINVAL,
              "grad_out, y and dy must be 16-byte aligned");
  if (T == 0) return MOE_OK;
  hipStream_t st = as_stream(stream);
  uint16_t* o = static_cast<uint16_t*>(dy);
  if (g_t == MOE_BF16 && y_t == MOE_BF16)
    hipLaunchKernelGGL((k_combine_bwd<uint16_t, uint16_t>), dim3(T), dim3(CBB_THREADS), 0, st, cp<uint16_t>(grad_out),
                       cp<uint16_t>(y), inv_row, topk_gate, topk_score, seg_offset, d, K, Nr, Ns, o, dgate, dz,
                       dz_row);
  else if (g_t == MOE_BF16)
    hipLaunchKernelGGL((k_combine_bwd<uint16_t, float>), dim3(T), dim3(CBB_THREADS), 0, st, cp<uint16_t>(grad_out),
                       cp<float>(y), inv_row, topk_gate, topk_score, seg_offset, d, K, Nr, Ns, o, dgate, dz, dz_row);
  else if (y_t == MOE_BF16)
    hipLaunchKernelGGL((k_combine_bwd<float, uint16_t>), dim3(T), dim3(CBB_THREADS), 0, st, cp<float>(grad_out),
                       cp<uint16_t>(y), inv_row, topk_gate, topk_score, seg_offset, d, K, Nr, Ns, o, dgate, dz,
                       dz_row);
  else
    hipLaunchKernelGGL((k_combine_bwd<float, float>), dim3(T), dim3(CBB_THREADS), 0, st, cp<float>(grad_out),
                       cp<float>(y), inv_row, topk_gate, topk_score, seg_offset, d, K, Nr, Ns, o, dgate, dz, dz_row);
  return launch_status("moe_combine_backward");
}

// Workspace of the bf16 backward: [da | db] bf16 [P, 2I], then the wgrad's
// expert-to-XCD deal (8 x ceil(Nr / 8) int32).
static size_t deal_bytes(int Nr) { return (size_t)8 * ((Nr + 7) / 8) * 4; }
static size_t bwd_deal_offset(size_t P, int I) { return (P * (size_t)(2 * I) * 2 + 255) / 256 * 256; }

size_t gemm_backward_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  if (T < 0 || d < 1 || I < 1 || Nr < 1 || Ns < 0 || K < 1 || tile_m < 1) return 0;
  return bwd_deal_offset(permute_rows(T, K, Nr, Ns, tile_m), I) + deal_bytes(Nr);
}

moe_status expert_gemm_backward(const void* x, const void* w13, const void* w2, const void* h, const void* ab,
                                const void* dy, int T, int K, int Nr, int Ns, int d, int I, int tile_m,
                                const int32_t* seg_offset, const int32_t* row_token, const int32_t* tile_map,
                                const int32_t* n_tiles, void* ws, size_t ws_bytes, void* dx, void* dw13, void* dw2,
                                moe_dtype dw_t, void* stream) {
  const moe_status cs = check_layer(T, K, Nr, Ns, d, I, tile_m);
  if (cs != MOE_OK) return cs;
  MOE_REQUIRE(dw_t == MOE_F32 || dw_t == MOE_BF16, MOE_EINVAL, "dw_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(w13 && w2 && seg_offset && row_token && tile_map && n_tiles && dw13 && dw2, MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(T == 0 || (x && h && ab && dy && dx), MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(aligned16(x) && aligned16(w13) && aligned16(w2) && aligned16(h) && aligned16(ab) && aligned16(dy) &&
                  aligned16(ws) && aligned16(dx) && aligned16(dw13) && aligned16(dw2),
              MOE_EINVAL, "data tensors and ws must be 16-byte aligned");
  MOE_REQUIRE(ffn_bwd_ok(d, I), MOE_EUNSUPPORTED, "backward needs d % 256 == 0 and I % 128 == 0");
  const size_t P = permute_rows(T, K, Nr, Ns, tile_m);
  MOE_REQUIRE(fits31((unsigned long long)T * d * 2) && fits31((unsigned long long)P * d * 2) &&
                  fits31((unsigned long long)P * 2 * I * 2) && fits31((unsigned long long)2 * I * d * 2),
              MOE_EUNSUPPORTED, "backward: operand of 2 GiB or more");
  MOE_REQUIRE(ws && ws_bytes >= gemm_backward_workspace_bytes(T, K, Nr, Ns, d, I, tile_m), MOE_EWORKSPACE,
              "workspace smaller than moe_gemm_backward_workspace_bytes");
  const int tiles_max = (int)permute_tiles_max(T, K, Nr, Ns, tile_m);
  launch_ffn_bwd_bf16(cp<uint16_t>(x), cp<uint16_t>(w13), cp<uint16_t>(w2), cp<uint16_t>(h), cp<uint16_t>(ab),
                      cp<uint16_t>(dy), seg_offset, row_token, tile_map, n_tiles, tiles_max, T, (long long)P, d, I, Nr,
                      Ns, static_cast<uint16_t*>(ws),
                      reinterpret_cast<int*>(static_cast<uint8_t*>(ws) + bwd_deal_offset(P, I)),
                      static_cast<uint16_t*>(dx), dw13, dw2, dw_t == MOE_F32, as_stream(stream));
  return launch_status("moe_expert_gemm_backward");
}

// Workspace of the E4M3-dgrad backward: [da | db] bf16, its E4M3 codes, the
// codes of dy, then the fp32 1x128 scales of both, each part 256-byte aligned.
struct W8Ws {
  size_t dab, dabq, dyq, dabs, dys, deal, total;
  W8Ws(size_t P, int d, int I, int Nr) {
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    dab = 0;
    dabq = dab + up(P * 2 * I * 2);
    dyq = dabq + up(P * 2 * I);
    dabs = dyq + up(P * d);
    dys = dabs + up(P * (2 * I / 128) * 4);
    deal = dys + up(P * (d / 128) * 4);
    total = deal + deal_bytes(Nr);
  }
};

size_t gemm_backward_w8_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  if (T < 0 || d < 128 || I < 64 || Nr < 1 || Ns < 0 || K < 1 || tile_m < 1) return 0;
  return W8Ws(permute_rows(T, K, Nr, Ns, tile_m), d, I, Nr).total;
}

// Workspace of the all-E4M3 backward: W8Ws, then the run codes of h, of the
// gathered x, of dy and of [da | db], the four run-scale arrays [runs, C]
// (dy, h, [da | db], x) and run_offset [Nr + Ns + 1].
struct F8Ws {
  W8Ws w8;
  size_t hr, xr, dyr, dabr, dyrs, hrs, dabrs, xrs, run_offset, total;
  F8Ws(size_t P, int d, int I, int Nr, int Ns) : w8(P, d, I, Nr) {
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    const size_t runs = (size_t)quantize_runs_max((long long)P, Nr + Ns);
    hr = up(w8.total);
    xr = hr + up(P * I);
    dyr = xr + up(P * d);
    dabr = dyr + up(P * d);
    dyrs = dabr + up(P * 2 * I);
    hrs = dyrs + up(runs * d * 4);
    dabrs = hrs + up(runs * I * 4);
    xrs = dabrs + up(runs * 2 * I * 4);
    run_offset = xrs + up(runs * d * 4);
    total = run_offset + up((size_t)(Nr + Ns + 1) * 4);
  }
};

size_t gemm_backward_f8_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  if (T < 0 || d < 128 || I < 64 || Nr < 1 || Ns < 0 || K < 1 || tile_m < 1) return 0;
  return F8Ws(permute_rows(T, K, Nr, Ns, tile_m), d, I, Nr, Ns).total;
}

// The argument checks of the E4M3 backward calls; P the permuted rows.
static moe_status check_backward_w8(const void* x, const uint8_t* w13, const float* w13_scale, const uint8_t* w2,
                                    const float* w2_scale, const void* h, const void* ab, const void* dy, int T,
                                    int K, int Nr, int Ns, int d, int I, int tile_m, const int32_t* seg_offset,
                                    const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles,
                                    void* ws, void* dx, void* dw13, void* dw2, moe_dtype dw_t, size_t& P) {
  const moe_status cs = check_layer(T, K, Nr, Ns, d, I, tile_m);
  if (cs != MOE_OK) return cs;
  MOE_REQUIRE(dw_t == MOE_F32 || dw_t == MOE_BF16, MOE_EINVAL, "dw_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(w13 && w13_scale && w2 && w2_scale && seg_offset && row_token && tile_map && n_tiles && dw13 && dw2,
              MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(T == 0 || (x && h && ab && dy && dx), MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(aligned16(x) && aligned16(w13) && aligned16(w2) && aligned16(h) && aligned16(ab) && aligned16(dy) &&
                  aligned16(ws) && aligned16(dx) && aligned16(dw13) && aligned16(dw2),
              MOE_EINVAL, "data tensors and ws must be 16-byte aligned");
  MOE_REQUIRE(ffn_bwd_w8_ok(d, I), MOE_EUNSUPPORTED,
              "E4M3 backward needs d % 256 == 0, I % 128 == 0, d <= 16384 and I <= 8192");
  P = permute_rows(T, K, Nr, Ns, tile_m);
  MOE_REQUIRE(fits31((unsigned long long)T * d * 2) && fits31((unsigned long long)P * d * 2) &&
                  fits31((unsigned long long)P * 2 * I * 2) && fits31((unsigned long long)2 * I * d * 2),
              MOE_EUNSUPPORTED, "backward: operand of 2 GiB or more");
  return MOE_OK;
}

moe_status expert_gemm_backward_f8(const void* x, const uint8_t* w13, const float* w13_scale, const uint8_t* w2,
                                   const float* w2_scale, const void* h, const void* ab, const void* dy, int T, int K,
                                   int Nr, int Ns, int d, int I, int tile_m, const int32_t* seg_offset,
                                   const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles,
                                   void* ws, size_t ws_bytes, void* dx, void* dw13, void* dw2, moe_dtype dw_t,
                                   void* stream) {
  size_t P = 0;
  const moe_status cs = check_backward_w8(x, w13, w13_scale, w2, w2_scale, h, ab, dy, T, K, Nr, Ns, d, I, tile_m,
                                          seg_offset, row_token, tile_map, n_tiles, ws, dx, dw13, dw2, dw_t, P);
  if (cs != MOE_OK) return cs;
  const size_t runs = (size_t)quantize_runs_max((long long)P, Nr + Ns);
  MOE_REQUIRE(fits31((unsigned long long)runs * d * 4) && fits31((unsigned long long)runs * 2 * I * 4),
              MOE_EUNSUPPORTED, "backward: operand of 2 GiB or more");
  const F8Ws L(P, d, I, Nr, Ns);
  MOE_REQUIRE(ws && ws_bytes >= L.total, MOE_EWORKSPACE, "workspace smaller than moe_gemm_backward_f8_workspace_bytes");
  const int tiles_max = (int)permute_tiles_max(T, K, Nr, Ns, tile_m);
  uint8_t* wb = static_cast<uint8_t*>(ws);
  auto f = [&](size_t o) { return reinterpret_cast<float*>(wb + o); };
  launch_ffn_bwd_f8(cp<uint16_t>(x), w13, w13_scale, w2, w2_scale, cp<uint16_t>(h), cp<uint16_t>(ab),
                    cp<uint16_t>(dy), seg_offset, row_token, tile_map, n_tiles, tiles_max, T, (long long)P, d, I, Nr,
                    Ns, reinterpret_cast<uint16_t*>(wb + L.w8.dab), wb + L.w8.dyq, f(L.w8.dys), wb + L.w8.dabq,
                    f(L.w8.dabs), wb + L.hr, wb + L.xr, wb + L.dyr, wb + L.dabr, f(L.dyrs), f(L.hrs), f(L.dabrs),
                    f(L.xrs),
                    reinterpret_cast<int32_t*>(wb + L.run_offset), reinterpret_cast<int*>(wb + L.w8.deal),
                    static_cast<uint16_t*>(dx), dw13, dw2, dw_t == MOE_F32, as_stream(stream));
  return launch_status("moe_expert_gemm_backward_f8");
}

moe_status expert_gemm_backward_w8(const void* x, const uint8_t* w13, const float* w13_scale, const uint8_t* w2,
                                   const float* w2_scale, const void* h, const void* ab, const void* dy, int T, int K,
                                   int Nr, int Ns, int d, int I, int tile_m, const int32_t* seg_offset,
                                   const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles,
                                   void* ws, size_t ws_bytes, void* dx, void* dw13, void* dw2, moe_dtype dw_t,
                                   void* stream) {
  size_t P = 0;
  const moe_status cs = check_backward_w8(x, w13, w13_scale, w2, w2_scale, h, ab, dy, T, K, Nr, Ns, d, I, tile_m,
                                          seg_offset, row_token, tile_map, n_tiles, ws, dx, dw13, dw2, dw_t, P);
  if (cs != MOE_OK) return cs;
  const W8Ws L(P, d, I, Nr);
  MOE_REQUIRE(ws && ws_bytes >= L.total, MOE_EWORKSPACE, "workspace smaller than moe_gemm_backward_w8_workspace_bytes");
  // T == 0 still launches: the weight-gradient kernels write the zeros of
  // the experts without rows (every expert here)
  const int tiles_max = (int)permute_tiles_max(T, K, Nr, Ns, tile_m);
  uint8_t* wb = static_cast<uint8_t*>(ws);
  launch_ffn_bwd_w8(cp<uint16_t>(x), w13, w13_scale, w2, w2_scale, cp<uint16_t>(h), cp<uint16_t>(ab),
                    cp<uint16_t>(dy), seg_offset, row_token, tile_map, n_tiles, tiles_max, T, (long long)P, d, I, Nr,
                    Ns, reinterpret_cast<uint16_t*>(wb + L.dab), wb + L.dyq, reinterpret_cast<float*>(wb + L.dys),
                    wb + L.dabq, reinterpret_cast<float*>(wb + L.dabs), reinterpret_cast<int*>(wb + L.deal),
                    static_cast<uint16_t*>(dx), dw13, dw2, dw_t == MOE_F32, as_stream(stream));
  return launch_status("moe_expert_gemm_backward_w8");
}

moe_status route_backward(const void* grad_out, moe_dtype g_t, const void* dx, const void* u, moe_dtype u_t,
                          const float* centroids, const int32_t* topk_idx, const int32_t* inv_row, const float* dz,
                          const float* dz_row, const int32_t* seg_offset, const int32_t* row_token, int T, int d,
                          int K, int Nr, int Ns, void* du, moe_dtype du_t, float* de, void* stream) {
  MOE_REQUIRE(T >= 0 && d >= 8 && d % 8 == 0, MOE_EINVAL, "need T >= 0 and d a positive multiple of 8");
  MOE_REQUIRE(Nr >= 1 && Ns >= 0 && Nr + Ns <= MOE_MAX_EXPERTS, MOE_EINVAL, "expert counts out of range");
  MOE_REQUIRE(K >= 1 && K <= MOE_MAX_K && K <= Nr, MOE_EINVAL, "K out of range");
  MOE_REQUIRE(g_t == MOE_F32 || g_t == MOE_BF16, MOE_EINVAL, "g_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(u_t == MOE_F32 || u_t == MOE_BF16, MOE_EINVAL, "u_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(du_t == MOE_F32 || du_t == MOE_BF16, MOE_EINVAL, "du_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(centroids && seg_offset && row_token && de, MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(T == 0 || (grad_out && dx && u && topk_idx && inv_row && dz && dz_row && du), MOE_EINVAL,
              "NULL pointer");
  MOE_REQUIRE(aligned16(grad_out) && aligned16(dx) && aligned16(u) && aligned16(centroids) && aligned16(du) &&
                  aligned16(de),
              MOE_EINVAL, "grad_out, dx, u, centroids, du and de must be 16-byte aligned");
  hipStream_t st = as_stream(stream);
  const dim3 gi((unsigned)Nr, (unsigned)ceil_div(d, CG_COLS));
  if (u_t == MOE_BF16)
    hipLaunchKernelGGL((k_centroid_grad<uint16_t>), gi, dim3(CG_THREADS), 0, st, cp<uint16_t>(u), seg_offset,
                       row_token, dz_row, d, de);
  else
    hipLaunchKernelGGL((k_centroid_grad<float>), gi, dim3(CG_THREADS), 0, st, cp<float>(u), seg_offset, row_token,
                       dz_row, d, de);
  if (T > 0) {
    const dim3 gt((unsigned)T, (unsigned)ceil_div(d, IG_COLS));
    const uint16_t* dxb = cp<uint16_t>(dx);
    const int key = (g_t == MOE_BF16) * 2 + (du_t == MOE_BF16);
    switch (key) {
      case 0:
        hipLaunchKernelGGL((k_input_grad<float, float>), gt, dim3(IG_THREADS), 0, st, cp<float>(grad_out), dxb,
                           centroids, topk_idx, inv_row, dz, seg_offset, d, K, Nr, Ns, static_cast<float*>(du));
        break;
      case 1:
        hipLaunchKernelGGL((k_input_grad<float, uint16_t>), gt, dim3(IG_THREADS), 0, st, cp<float>(grad_out), dxb,
                           centroids, topk_idx, inv_row, dz, seg_offset, d, K, Nr, Ns, static_cast<uint16_t*>(du));
        break;
      case 2:
        hipLaunchKernelGGL((k_input_grad<uint16_t, float>), gt, dim3(IG_THREADS), 0, st, cp<uint16_t>(grad_out), dxb,
                           centroids, topk_idx, inv_row, dz, seg_offset, d, K, Nr, Ns, static_cast<float*>(du));
        break;
      default:
        hipLaunchKernelGGL((k_input_grad<uint16_t, uint16_t>), gt, dim3(IG_THREADS), 0, st, cp<uint16_t>(grad_out),
                           dxb, centroids, topk_idx, inv_row, dz, seg_offset, d, K, Nr, Ns,
                           static_cast<uint16_t*>(du));
        break;
    }
  }
  return launch_status("moe_route_backward");
}

}  // namespace moe
