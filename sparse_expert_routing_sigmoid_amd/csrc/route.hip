// moe_route: sigmoid affinities, bias-steered top-K, normalised gates, loads.
//
// Follows the "DeepSeek-V3 Technical Report" reading guide (xyznot.com),
// Method section 2: s_{i,t} = Sigmoid(u_t . e_i) (affinity sentence);
// selection on s + b, kept value s (gate equation); gates are the kept
// values normalised over the selection; ties go to the lower expert index.
//
// Kernels:
//   k_router_logits_mfma  (bf16 u, Nr <= 256) z = u . e on bf16 MFMA with e
//                    split exactly into three bf16 parts, 128 or 256 tokens
//                    per block; K split over blocks into partial sums added
//                    in a fixed order later.
//   k_router_logits  (fp32 u, or other shapes) z[t, i] = u_t . e_i in fp32 on
//                    the vector ALUs, LDS tiles of 64 tokens x 64 experts;
//                    every 32-wide K chunk is summed into its own partial
//                    before it joins the running sum, which keeps the fp32
//                    error of a d = 7168 dot product near 1e-7.
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

// ---- bf16 activations: logits on MFMA with a three-way bf16 split of e.
// e = e1 + e2 + e3 with e1 = bf16(e), e2 = bf16(e - e1), e3 = bf16(e - e1 - e2)
// (each remainder is exact in fp32), so e is represented to about 2^-27
// relative, every product u * e_k is exact in fp32 and the MFMA sums them in
// fp32.  The split is made once per call into the workspace.
typedef __bf16 bf16x8_r __attribute__((ext_vector_type(8)));
typedef float f32x16_r __attribute__((ext_vector_type(16)));

__global__ void k_split_centroids(const float* __restrict__ e, long long n, uint16_t* __restrict__ e3) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = e[i];
  const __bf16 a = static_cast<__bf16>(v);
  const float r1 = v - static_cast<float>(a);
  const __bf16 b = static_cast<__bf16>(r1);
  const float r2 = r1 - static_cast<float>(b);
  const __bf16 c = static_cast<__bf16>(r2);
  e3[i] = __builtin_bit_cast(uint16_t, a);
  e3[n + i] = __builtin_bit_cast(uint16_t, b);
  e3[2 * n + i] = __builtin_bit_cast(uint16_t, c);
}

constexpr int RM_TE = 256;              // experts per block (all, Nr <= 256)
constexpr int RM_BK = 32;               // K per stage
constexpr int RM_ROW = RM_BK * 2;       // LDS row bytes: four 16-byte chunks
constexpr int RM_BROWS = 3 * RM_TE;     // B rows: e1, e2, e3 of 256 experts

// Tokens per block: 256 when there are enough tokens to fill the chip with
// them (the centroid rows, the bulk of each stage, then serve twice as many
// tokens), else 128.
inline int router_tile_tokens(int T) { return T >= 4096 ? 256 : 128; }

// LDS offset of 16-byte chunk c of row r: the chunk index is XORed with
// (r >> 1) & 3, so the 8 rows one fragment read touches at a time (row pairs
// 128 bytes apart) fall on distinct banks.
__device__ __forceinline__ int rm_off(int r, int c) { return r * RM_ROW + ((c ^ ((r >> 1) & 3)) << 4); }

// Partial logits zp[ks][t][i] = sum over the ks-th K chunk of u[t,k] * e[i,k].
// Grid (T / TT, KS); 256 threads = 4 waves; wave w covers all TT tokens of
// the block and experts 64 w .. 64 w + 63 (TT/32 x 2 MFMA 32x32 tiles),
// running the three bf16 parts of e into the same fp32 accumulators.
// Operands are staged through registers into a double-buffered LDS tile.
template <int TT>
__global__ __launch_bounds__(256) void k_router_logits_mfma(const uint16_t* __restrict__ u,
                                                            const uint16_t* __restrict__ e3, int T, int d, int Nr,
                                                            int kchunk, float* __restrict__ zp) {
  constexpr int MI = TT / 32;                          // 32-token MFMA tiles
  constexpr int QA = TT * 4 / 256;                     // A chunks per thread and stage
  constexpr int QB = RM_BROWS * 4 / 256;               // B chunks per thread and stage
  constexpr int SBYTES = (TT + RM_BROWS) * RM_ROW;     // one stage
  extern __shared__ __attribute__((aligned(16))) uint8_t rs[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * TT;
  const int ks = blockIdx.y;
  const int k_begin = ks * kchunk;
  const int nk = kchunk / RM_BK;
  const long long nE = (long long)Nr * d;
  uint4 ra[QA], rb[QB];
  auto gload = [&](int stage) {
    const int kofs = k_begin + stage * RM_BK;
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int c = tid + 256 * q, r = c >> 2, ch = c & 3;
      const int t = t0 + r;
      ra[q] = t < T ? *reinterpret_cast<const uint4*>(u + (long long)t * d + kofs + ch * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int c = tid + 256 * q, r = c >> 2, ch = c & 3;
      const int part = r / RM_TE, ex = r % RM_TE;
      rb[q] = ex < Nr ? *reinterpret_cast<const uint4*>(e3 + part * nE + (long long)ex * d + kofs + ch * 8)
                      : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](uint8_t* sb) {
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int c = tid + 256 * q, r = c >> 2, ch = c & 3;
      *reinterpret_cast<uint4*>(sb + rm_off(r, ch)) = ra[q];
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int c = tid + 256 * q, r = c >> 2, ch = c & 3;
      *reinterpret_cast<uint4*>(sb + rm_off(TT + r, ch)) = rb[q];
    }
  };
  f32x16_r acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  const int e0 = wave * 64;  // this wave's experts
  gload(0);
  lstore(rs);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    uint8_t* cur = rs + (s & 1) * SBYTES;
    if (s + 1 < nk) gload(s + 1);
#pragma unroll
    for (int kk = 0; kk < RM_BK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      bf16x8_r af[MI];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        af[i] = __builtin_bit_cast(bf16x8_r, *reinterpret_cast<const uint4*>(cur + rm_off(i * 32 + (lane & 31), c)));
#pragma unroll
      for (int part = 0; part < 3; ++part)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x8_r bfr = __builtin_bit_cast(
              bf16x8_r, *reinterpret_cast<const uint4*>(
                            cur + rm_off(TT + part * RM_TE + e0 + j * 32 + (lane & 31), c)));
#pragma unroll
          for (int i = 0; i < MI; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr, acc[i][j], 0, 0, 0);
        }
    }
    if (s + 1 < nk) lstore(rs + ((s + 1) & 1) * SBYTES);
    __syncthreads();
  }
  float* zo = zp + (long long)ks * T * Nr;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int t = t0 + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        const int ex = e0 + j * 32 + (lane & 31);
        if (t < T && ex < Nr) zo[(long long)t * Nr + ex] = acc[i][j][q];
      }
}

// K-split count of the MFMA router for T tokens and hidden size d (0 = the
// MFMA router does not apply): enough blocks to fill the chip (one per CU
// with 256-token tiles, whose LDS takes a whole CU; two rounds with 128),
// each chunk a multiple of the stage width.
int router_ksplit(int T, int d, int Nr) {
  if (Nr > RM_TE || d % RM_BK != 0) return 0;
  const int tt = router_tile_tokens(T);
  const int tiles = (T + tt - 1) / tt;
  const int target = tt == 256 ? 256 : 512;
  int ks = 1;
  while (ks < 32 && tiles * ks < target && d % (RM_BK * ks * 2) == 0) ks *= 2;
  return ks;
}

template <int TT>
moe_status launch_router_mfma(const uint16_t* u, const uint16_t* e3, int T, int d, int Nr, int ks, float* z,
                              hipStream_t st) {
  dim3 grid((T + TT - 1) / TT, ks);
  const size_t lds = 2 * (size_t)(TT + RM_BROWS) * RM_ROW;
  // The dynamic LDS limit is raised on every call (for the current device;
  // idempotent and cheap), so the library keeps no per-process state for it.
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_router_logits_mfma<TT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
    set_error("moe_route: cannot raise the LDS limit of the router kernel");
    return MOE_EHIP;
  }
  hipLaunchKernelGGL(k_router_logits_mfma<TT>, grid, dim3(256), lds, st, u, e3, T, d, Nr, d / ks, z);
  return MOE_OK;
}

__global__ void k_zero_i32(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// EPL = experts per lane (Nr <= 64 * EPL).  One wave per token; each wave
// takes tpw consecutive tokens.  Loads are counted in an LDS histogram and
// added to expert_load once per block, which keeps the global atomics on a
// popular expert few.
template <int EPL>
__global__ __launch_bounds__(256) void k_route_select(const float* __restrict__ z, int nparts,
                                                      const float* __restrict__ bias, int T, int Nr, int K, int tpw,
                                                      int32_t* __restrict__ topk_idx,
                                                      float* __restrict__ topk_gate, float* __restrict__ topk_score,
                                                      int32_t* __restrict__ load) {
  __shared__ int s_hist[64 * EPL];
  for (int i = threadIdx.x; i < Nr; i += blockDim.x) s_hist[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int t_first = (blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)) * tpw;
  for (int t = t_first; t < t_first + tpw && t < T; ++t) {
  float s[EPL];
  unsigned long long key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int i = lane + 64 * j;
    if (i < Nr) {
      // partial sums added in the fixed order 0, 1, ..., nparts - 1; loaded
      // eight at a time so their latencies overlap
      const float* zi = z + (long long)t * Nr + i;
      const long long ps = (long long)T * Nr;
      float zz;
      int p;
      if (nparts >= 8) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = zi[q * ps];
        zz = v[0];
#pragma unroll
        for (int q = 1; q < 8; ++q) zz += v[q];
        for (p = 8; p + 8 <= nparts; p += 8) {
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = zi[(p + q) * ps];
#pragma unroll
          for (int q = 0; q < 8; ++q) zz += v[q];
        }
      } else {
        zz = zi[0];
        p = 1;
      }
      for (; p < nparts; ++p) zz += zi[p * ps];
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
    atomicAdd(&s_hist[my_idx], 1);
  }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < Nr; i += blockDim.x)
    if (s_hist[i]) atomicAdd(&load[i], s_hist[i]);
}

template <int EPL>
void launch_select(const float* z, int nparts, const float* bias, int T, int Nr, int K, int32_t* idx, float* gate,
                   float* score, int32_t* load, hipStream_t st) {
  const int waves_per_block = 4;
  const int tpw = T >= 16384 ? 8 : (T >= 4096 ? 4 : 1);  // tokens per wave
  const int per_block = waves_per_block * tpw;
  dim3 grid((T + per_block - 1) / per_block);
  hipLaunchKernelGGL(k_route_select<EPL>, grid, dim3(64 * waves_per_block), 0, st, z, nparts, bias, T, Nr, K, tpw,
                     idx, gate, score, load);
}

}  // namespace

// Workspace: partial logits [KS][T][Nr] fp32 (KS = 1 on the fp32 path),
// then the bf16 split of the centroids [3][Nr][d] for the MFMA path.
size_t route_workspace_bytes(int T, int d, int Nr) {
  if (T < 0 || Nr < 0 || d < 0) return 0;
  const int ks = router_ksplit(T, d, Nr);
  const size_t z = (size_t)(ks > 0 ? ks : 1) * (size_t)T * (size_t)Nr * sizeof(float);
  const size_t split = (size_t)3 * Nr * d * 2;
  return ((z + 255) / 256) * 256 + split + 256;
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
  MOE_REQUIRE(aligned16(u) && aligned16(centroids) && aligned16(ws), MOE_EINVAL,
              "u, centroids and ws must be 16-byte aligned");
  MOE_REQUIRE(T == 0 || (ws && ws_bytes >= route_workspace_bytes(T, d, Nr)), MOE_EWORKSPACE,
              "workspace smaller than moe_route_workspace_bytes");
  hipStream_t st = as_stream(stream);
  hipLaunchKernelGGL(k_zero_i32, dim3((Nr + 255) / 256), dim3(256), 0, st, expert_load, Nr);
  if (T > 0) {
    float* z = static_cast<float*>(ws);
    int nparts = 1;
    const int ks = u_t == MOE_BF16 ? router_ksplit(T, d, Nr) : 0;
    if (ks > 0) {
      const size_t zbytes = (size_t)ks * T * Nr * sizeof(float);
      uint16_t* e3 = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + ((zbytes + 255) / 256) * 256);
      const long long n = (long long)Nr * d;
      hipLaunchKernelGGL(k_split_centroids, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, centroids, n, e3);
      const moe_status ls = router_tile_tokens(T) == 256
                                ? launch_router_mfma<256>(static_cast<const uint16_t*>(u), e3, T, d, Nr, ks, z, st)
                                : launch_router_mfma<128>(static_cast<const uint16_t*>(u), e3, T, d, Nr, ks, z, st);
      if (ls != MOE_OK) return ls;
      nparts = ks;
    } else {
      dim3 grid((T + LG_TT - 1) / LG_TT, (Nr + LG_TE - 1) / LG_TE);
      if (u_t == MOE_F32)
        hipLaunchKernelGGL(k_router_logits<float>, grid, dim3(256), 0, st, static_cast<const float*>(u), centroids, T,
                           d, Nr, z);
      else
        hipLaunchKernelGGL(k_router_logits<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(u),
                           centroids, T, d, Nr, z);
    }
    if (Nr <= 64)
      launch_select<1>(z, nparts, bias, T, Nr, K, topk_idx, topk_gate, topk_score, expert_load, st);
    else if (Nr <= 256)
      launch_select<4>(z, nparts, bias, T, Nr, K, topk_idx, topk_gate, topk_score, expert_load, st);
    else
      launch_select<16>(z, nparts, bias, T, Nr, K, topk_idx, topk_gate, topk_score, expert_load, st);
  }
  return launch_status("moe_route");
}

}  // namespace moe
