// moe_permute: stable counting sort of the (token, slot) pairs by expert into
// padded, expert-contiguous segments, plus the row-tile map of the GEMM.
//
// Every routed expert's segment lists the tokens that selected it in
// increasing token order; shared expert j's segment lists every token (the
// shared sum of the combine equation in the "DeepSeek-V3 Technical Report"
// reading guide, Method section 2).  No token is dropped, so a segment can
// hold all T tokens.
//
// Three kernels, no host synchronisation, deterministic output:
//   k_perm_count    per block of 256 tokens, per-expert counts (LDS atomics;
//                   a count does not depend on the order of the adds)
//   k_perm_scan     one block: per-expert exclusive scan over the blocks,
//                   padded segment sizes, segment offsets, tile map, -1 fill
//                   of the padding rows
//   k_perm_scatter  per block: stable rank of every (t, k) inside its block
//                   from per-wave 64-bit masks (popcount of the lower lanes
//                   that chose the same expert), then the row of (t, k).
#include "common.h"

#include <mutex>

namespace moe {

namespace {

constexpr int PB_TOK = 256;    // tokens per block (one per thread)
constexpr int PB_WAVES = PB_TOK / 64;

__global__ __launch_bounds__(PB_TOK) void k_perm_count(const int32_t* __restrict__ idx, int T, int K, int Nr,
                                                       int32_t* __restrict__ counts) {
  extern __shared__ int32_t cnt[];
  for (int e = threadIdx.x; e < Nr; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * PB_TOK + threadIdx.x;
  if (t < T)
    for (int k = 0; k < K; ++k) atomicAdd(&cnt[idx[(long long)t * K + k]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < Nr; e += blockDim.x) counts[(long long)blockIdx.x * Nr + e] = cnt[e];
}

// One block of 1024 threads; thread e owns segment e (E = Nr + Ns <= 1024).
__global__ __launch_bounds__(1024) void k_perm_scan(int32_t* __restrict__ counts, int nblk, int T, int Nr, int Ns,
                                                    int tile_m, int32_t* __restrict__ seg_offset,
                                                    int32_t* __restrict__ row_token, int32_t* __restrict__ tile_map,
                                                    int32_t* __restrict__ n_tiles, int32_t* __restrict__ seg_load) {
  __shared__ long long s_rows[1024];
  __shared__ int s_tiles[1024];
  const int e = threadIdx.x;
  const int E = Nr + Ns;
  int load = 0;
  if (e < Nr) {
    for (int b = 0; b < nblk; ++b) {
      int32_t* c = counts + (long long)b * Nr + e;
      const int v = *c;
      *c = load;          // becomes the block's base inside the segment
      load += v;
    }
  } else if (e < E) {
    load = T;
  }
  const int padded = e < E ? (int)(ceil_div(load, tile_m) * tile_m) : 0;
  const int ntile = (int)ceil_div(padded, MOE_TILE_ROWS);
  s_rows[e] = padded;
  s_tiles[e] = ntile;
  __syncthreads();
  // Inclusive Hillis-Steele scans over the 1024 segments.
  for (int off = 1; off < 1024; off <<= 1) {
    const long long r = e >= off ? s_rows[e - off] : 0;
    const int tl = e >= off ? s_tiles[e - off] : 0;
    __syncthreads();
    s_rows[e] += r;
    s_tiles[e] += tl;
    __syncthreads();
  }
  const int row0 = (int)(s_rows[e] - padded);
  const int tile0 = s_tiles[e] - ntile;
  if (e < E) {
    seg_offset[e] = row0;
    seg_load[e] = load;
    for (int r = load; r < padded; ++r) row_token[row0 + r] = -1;
    for (int j = 0; j < ntile; ++j) {
      int32_t* m = tile_map + 4LL * (tile0 + j);
      const int rows = padded - j * MOE_TILE_ROWS < MOE_TILE_ROWS ? padded - j * MOE_TILE_ROWS : MOE_TILE_ROWS;
      m[0] = e;
      m[1] = row0 + j * MOE_TILE_ROWS;
      m[2] = rows;
      const int real = load - j * MOE_TILE_ROWS;  // token rows come first, padding last
      m[3] = real < 0 ? 0 : (real > rows ? rows : real);
    }
  }
  if (e == E - 1) {
    seg_offset[E] = (int)s_rows[e];
    *n_tiles = s_tiles[e];
  }
}

__global__ __launch_bounds__(PB_TOK) void k_perm_scatter(const int32_t* __restrict__ idx, int T, int K, int Nr, int Ns,
                                                         const int32_t* __restrict__ base,
                                                         const int32_t* __restrict__ seg_offset,
                                                         int32_t* __restrict__ row_token, int32_t* __restrict__ inv_row,
                                                         long long P_max) {
  extern __shared__ unsigned long long masks[];  // [PB_WAVES][Nr]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < PB_WAVES * Nr; i += blockDim.x) masks[i] = 0ull;
  __syncthreads();
  const int t = blockIdx.x * PB_TOK + tid;
  int ex[MOE_MAX_K];
#pragma unroll
  for (int k = 0; k < MOE_MAX_K; ++k) ex[k] = 0;
  if (t < T) {
#pragma unroll
    for (int k = 0; k < MOE_MAX_K; ++k)
      if (k < K) {
        ex[k] = idx[(long long)t * K + k];
        atomicOr(&masks[wave * Nr + ex[k]], 1ull << lane);
      }
  }
  __syncthreads();
  if (t < T) {
    const unsigned long long lower = (1ull << lane) - 1ull;
#pragma unroll
    for (int k = 0; k < MOE_MAX_K; ++k)
      if (k < K) {
        const int e = ex[k];
        int r = __popcll(masks[wave * Nr + e] & lower);
        for (int w = 0; w < wave; ++w) r += __popcll(masks[w * Nr + e]);
        const int row = seg_offset[e] + base[(long long)blockIdx.x * Nr + e] + r;
        row_token[row] = t;
        inv_row[(long long)t * K + k] = row;
      }
    for (int j = 0; j < Ns; ++j) row_token[seg_offset[Nr + j] + t] = t;
  }
  // Rows past the last segment are padding as well.
  const long long used = seg_offset[Nr + Ns];
  for (long long r = used + (long long)blockIdx.x * blockDim.x + tid; r < P_max; r += (long long)gridDim.x * blockDim.x)
    row_token[r] = -1;
}

}  // namespace

size_t permute_rows(int T, int K, int Nr, int Ns, int tile_m) {
  if (T < 0 || K < 0 || Nr < 0 || Ns < 0 || tile_m < 1) return 0;
  return (size_t)T * K + (size_t)Ns * T + (size_t)(Nr + Ns) * (tile_m - 1);
}

size_t permute_tiles_max(int T, int K, int Nr, int Ns, int tile_m) {
  const size_t P = permute_rows(T, K, Nr, Ns, tile_m);
  return P / MOE_TILE_ROWS + (size_t)(Nr + Ns) + 1;
}

size_t permute_workspace_bytes(int T, int K, int Nr, int Ns) {
  (void)K;
  if (T < 0 || Nr < 0 || Ns < 0) return 0;
  const size_t nblk = (size_t)ceil_div(T, PB_TOK);
  return (nblk * Nr + (size_t)(Nr + Ns) + 64) * sizeof(int32_t);
}

moe_status permute(const int32_t* topk_idx, int T, int K, int Nr, int Ns, int tile_m, int32_t* seg_offset,
                   int32_t* row_token, int32_t* inv_row, int32_t* tile_map, int32_t* n_tiles, void* ws,
                   size_t ws_bytes, void* stream) {
  MOE_REQUIRE(T >= 0, MOE_EINVAL, "T < 0");
  MOE_REQUIRE(Nr >= 1 && Ns >= 0 && Nr + Ns <= MOE_MAX_EXPERTS, MOE_EINVAL, "expert counts out of range");
  MOE_REQUIRE(K >= 1 && K <= MOE_MAX_K && K <= Nr, MOE_EINVAL, "K out of range");
  MOE_REQUIRE(tile_m >= 1 && tile_m <= MOE_TILE_ROWS && (tile_m & (tile_m - 1)) == 0, MOE_EINVAL,
              "tile_m must be a power of two in [1, MOE_TILE_ROWS]");
  MOE_REQUIRE(seg_offset && row_token && tile_map && n_tiles, MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(T == 0 || (topk_idx && inv_row), MOE_EINVAL, "NULL pointer");
  const long long P_max = (long long)permute_rows(T, K, Nr, Ns, tile_m);
  MOE_REQUIRE(P_max < (1LL << 31), MOE_EINVAL, "too many rows for int32 row indices");
  MOE_REQUIRE(ws && ws_bytes >= permute_workspace_bytes(T, K, Nr, Ns), MOE_EWORKSPACE,
              "workspace smaller than moe_permute_workspace_bytes");
  hipStream_t st = as_stream(stream);
  const int nblk = (int)ceil_div(T, PB_TOK);
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* seg_load = counts + (size_t)nblk * Nr;
  if (nblk > 0)
    hipLaunchKernelGGL(k_perm_count, dim3(nblk), dim3(PB_TOK), Nr * sizeof(int32_t), st, topk_idx, T, K, Nr, counts);
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, st, counts, nblk, T, Nr, Ns, tile_m, seg_offset, row_token,
                     tile_map, n_tiles, seg_load);
  const int sblk = nblk > 0 ? nblk : 1;
  hipLaunchKernelGGL(k_perm_scatter, dim3(sblk), dim3(PB_TOK), (size_t)PB_WAVES * Nr * sizeof(unsigned long long), st,
                     topk_idx, T, K, Nr, Ns, counts, seg_offset, row_token, inv_row, P_max);
  return launch_status("moe_permute");
}

// ------------------------------------------------- no-allocation variant --
// moe_permute_noalloc runs the same kernels with their workspace (per-block
// expert counts) in a device array of the library's own instead of a
// caller's buffer, for callers that cannot allocate.  Every word the kernels
// read there is written earlier in the same call, so nothing is cleared.
// Each GPU holds its own copy of the array until the process ends; its
// address on a device is looked up once, with that device current, and kept.
namespace {

constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(4) << 20;  // 4 MiB per GPU
constexpr int NOALLOC_MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

std::once_flag g_scratch_once[NOALLOC_MAX_DEVICES];
void* g_scratch_ptr[NOALLOC_MAX_DEVICES];
hipError_t g_scratch_err[NOALLOC_MAX_DEVICES];

}  // namespace

size_t permute_noalloc_scratch_bytes() { return NOALLOC_SCRATCH_BYTES; }

moe_status permute_noalloc(const int32_t* topk_idx, int T, int K, int Nr, int Ns, int tile_m, int32_t* seg_offset,
                           int32_t* row_token, int32_t* inv_row, int32_t* tile_map, int32_t* n_tiles, void* stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    set_error("moe_permute_noalloc: no current HIP device");
    return MOE_EHIP;
  }
  MOE_REQUIRE(dev < NOALLOC_MAX_DEVICES, MOE_EUNSUPPORTED, "device index beyond the library's limit");
  MOE_REQUIRE(T >= 0 && Nr >= 1 && Ns >= 0, MOE_EINVAL, "sizes out of range");
  MOE_REQUIRE(permute_workspace_bytes(T, K, Nr, Ns) <= NOALLOC_SCRATCH_BYTES, MOE_EWORKSPACE,
              "sizes need more than the 4 MiB of built-in scratch: (ceil(T/256)*Nr + Nr + Ns + 64) * 4 bytes; use "
              "moe_permute with a caller workspace");
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess) {
    set_error(std::string("moe_permute_noalloc: hipGetSymbolAddress of the scratch array: ") +
              hipGetErrorString(g_scratch_err[dev]));
    return MOE_EHIP;
  }
  return permute(topk_idx, T, K, Nr, Ns, tile_m, seg_offset, row_token, inv_row, tile_map, n_tiles,
                 g_scratch_ptr[dev], NOALLOC_SCRATCH_BYTES, stream);
}

}  // namespace moe
