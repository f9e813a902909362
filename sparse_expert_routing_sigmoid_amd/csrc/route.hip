// moe_route: sigmoid affinities, bias-steered top-K, normalised gates, loads.
//
// Follows the "DeepSeek-V3 Technical Report" reading guide (xyznot.com),
// Method section 2: s_{i,t} = Sigmoid(u_t . e_i) (affinity sentence);
// selection on s + b, kept value s (gate equation); gates are the kept
// values normalised over the selection; ties go to the lower expert index.
//
// Two kernels:
//   k_router_logits  z[t, i] = u_t . e_i in fp32 on the vector ALUs, LDS
//                    tiles of 64 tokens x 64 experts; every 32-wide K chunk
//                    is summed into its own partial before it joins the
//                    running sum, which keeps the fp32 error of a d = 7168
//                    dot product near 1e-7.
//   k_route_select   one wave per token: sigmoid, + bias, K rounds of a
//                    wave-wide max over 64-bit (order key of s+b, ~index)
//                    keys, gate normalisation, load count (integer atomics:
//                    the counts do not depend on their order).
#include "common.h"

namespace moe {

namespace {

constexpr int LG_TT = 64;   // tokens per block
constexpr int LG_TE = 64;   // experts per block
constexpr int LG_BK = 32;   // K chunk

template <typename UT>
__device__ __forceinline__ float load_act(const UT* p, long long i);
template <>
__device__ __forceinline__ float load_act<float>(const float* p, long long i) { return p[i]; }
template <>
__device__ __forceinline__ float load_act<uint16_t>(const uint16_t* p, long long i) { return bf16_to_f32(p[i]); }

template <typename UT>
__global__ __launch_bounds__(256) void k_router_logits(const UT* __restrict__ u, const float* __restrict__ e,
                                                       int T, int d, int Nr, float* __restrict__ z) {
  __shared__ float su[LG_BK][LG_TT + 4];
  __shared__ float se[LG_BK][LG_TE + 4];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * LG_TT;
  const int e0 = blockIdx.y * LG_TE;
  const int tr = tid / 16;  // 16 rows of 4 tokens
  const int ec = tid % 16;  // 16 cols of 4 experts
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += LG_BK) {
    // Stage a 64 x 32 slab of u and of e, transposed so the K index is the row.
    for (int i = tid; i < LG_TT * LG_BK; i += 256) {
      const int r = i / LG_BK, c = i % LG_BK;
      const int t = t0 + r, k = k0 + c;
      su[c][r] = (t < T && k < d) ? load_act(u, (long long)t * d + k) : 0.f;
      const int ex = e0 + r;
      se[c][r] = (ex < Nr && k < d) ? e[(long long)ex * d + k] : 0.f;
    }
    __syncthreads();
    float part[4][4] = {};
#pragma unroll 8
    for (int c = 0; c < LG_BK; ++c) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = su[c][tr * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = se[c][ec * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) part[i][j] = fmaf(a[i], b[j], part[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += part[i][j];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + tr * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ex = e0 + ec * 4 + j;
      if (ex < Nr) z[(long long)t * Nr + ex] = acc[i][j];
    }
  }
}

__global__ void k_zero_i32(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// EPL = experts per lane (Nr <= 64 * EPL).
template <int EPL>
__global__ __launch_bounds__(256) void k_route_select(const float* __restrict__ z, const float* __restrict__ bias,
                                                      int T, int Nr, int K, int32_t* __restrict__ topk_idx,
                                                      float* __restrict__ topk_gate, float* __restrict__ topk_score,
                                                      int32_t* __restrict__ load) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  float s[EPL];
  unsigned long long key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int i = lane + 64 * j;
    if (i < Nr) {
      const float zz = z[(long long)t * Nr + i];
      s[j] = 1.0f / (1.0f + expf(-zz));
      const float v = s[j] + bias[i];
      key[j] = (static_cast<unsigned long long>(float_order_key(v)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(i));
    } else {
      s[j] = 0.f;
      key[j] = 0ull;
    }
  }
  unsigned long long best = 0ull;
#pragma unroll
  for (int j = 0; j < EPL; ++j) best = key[j] > best ? key[j] : best;

  int my_idx = 0;
  float my_s = 0.f;
  for (int k = 0; k < K; ++k) {
    const unsigned long long w = wave_max_u64(best);
    const int i = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(w & 0xFFFFFFFFull));
    const int owner = i & 63;
    const int slot = i >> 6;
    float cand = 0.f;
    if (lane == owner) {
      best = 0ull;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        if (j == slot) {
          cand = s[j];
          key[j] = 0ull;
        }
        best = key[j] > best ? key[j] : best;
      }
    }
    const float sk = __shfl(cand, owner, 64);
    if (lane == k) {
      my_idx = i;
      my_s = sk;
    }
  }
  float sum = 0.f;
  for (int k = 0; k < K; ++k) sum += __shfl(my_s, k, 64);
  if (lane < K) {
    const long long o = (long long)t * K + lane;
    topk_idx[o] = my_idx;
    topk_gate[o] = my_s / sum;
    if (topk_score) topk_score[o] = my_s;
    atomicAdd(&load[my_idx], 1);
  }
}

template <int EPL>
void launch_select(const float* z, const float* bias, int T, int Nr, int K, int32_t* idx, float* gate, float* score,
                   int32_t* load, hipStream_t st) {
  const int waves_per_block = 4;
  dim3 grid((T + waves_per_block - 1) / waves_per_block);
  hipLaunchKernelGGL(k_route_select<EPL>, grid, dim3(64 * waves_per_block), 0, st, z, bias, T, Nr, K, idx, gate, score,
                     load);
}

}  // namespace

size_t route_workspace_bytes(int T, int d, int Nr) {
  (void)d;
  if (T < 0 || Nr < 0) return 0;
  return static_cast<size_t>(T) * static_cast<size_t>(Nr) * sizeof(float) + 256;
}

moe_status route(const void* u, moe_dtype u_t, const float* centroids, const float* bias, int T, int d, int Nr, int K,
                 int32_t* topk_idx, float* topk_gate, float* topk_score, int32_t* expert_load, void* ws,
                 size_t ws_bytes, void* stream) {
  MOE_REQUIRE(u_t == MOE_F32 || u_t == MOE_BF16, MOE_EINVAL, "u_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(T >= 0 && d >= 1 && d % 8 == 0, MOE_EINVAL, "need T >= 0 and d a positive multiple of 8");
  MOE_REQUIRE(Nr >= 1 && Nr <= MOE_MAX_EXPERTS, MOE_EINVAL, "Nr out of range");
  MOE_REQUIRE(K >= 1 && K <= MOE_MAX_K && K <= Nr, MOE_EINVAL, "K out of range");
  MOE_REQUIRE(expert_load != nullptr, MOE_EINVAL, "expert_load is NULL");
  MOE_REQUIRE(T == 0 || (u && centroids && bias && topk_idx && topk_gate), MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(T == 0 || (ws && ws_bytes >= route_workspace_bytes(T, d, Nr)), MOE_EWORKSPACE,
              "workspace smaller than moe_route_workspace_bytes");
  hipStream_t st = as_stream(stream);
  hipLaunchKernelGGL(k_zero_i32, dim3((Nr + 255) / 256), dim3(256), 0, st, expert_load, Nr);
  if (T > 0) {
    float* z = static_cast<float*>(ws);
    dim3 grid((T + LG_TT - 1) / LG_TT, (Nr + LG_TE - 1) / LG_TE);
    if (u_t == MOE_F32)
      hipLaunchKernelGGL(k_router_logits<float>, grid, dim3(256), 0, st, static_cast<const float*>(u), centroids, T, d,
                         Nr, z);
    else
      hipLaunchKernelGGL(k_router_logits<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(u), centroids,
                         T, d, Nr, z);
    if (Nr <= 64)
      launch_select<1>(z, bias, T, Nr, K, topk_idx, topk_gate, topk_score, expert_load, st);
    else if (Nr <= 256)
      launch_select<4>(z, bias, T, Nr, K, topk_idx, topk_gate, topk_score, expert_load, st);
    else
      launch_select<16>(z, bias, T, Nr, K, topk_idx, topk_gate, topk_score, expert_load, st);
  }
  return launch_status("moe_route");
}

}  // namespace moe
