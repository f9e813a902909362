// Persistent, XCD-aware grouped SwiGLU expert GEMM on bf16 MFMA (gfx950).
//
// The expert FFNs of the combine equation in the "DeepSeek-V3 Technical
// Report" reading guide (xyznot.com, Method section 2), in the SwiGLU form
// this library uses: h = SiLU(x W_gate^T) * (x W_up^T), y = h W_down^T.
//
// Work decomposition.  A work item is (row tile of the tile map, N tile).
// Phase A: N tile = 128 h columns = 128 gate rows + the 128 up rows of the
// same columns of W13.  Phase B: N tile = 256 columns of y (rows of W2).
// N tile n belongs to XCD n % 8, so every weight byte is fetched by one XCD
// only and all row tiles of an expert that share an N tile meet in that
// XCD's L2.  The kernel is persistent: 8 * (CUs / 8) blocks, block b runs on
// XCD b % 8 (workgroups are dealt to XCDs round robin) and pulls items of its
// XCD from a per-XCD atomic counter, in (row tile, N tile) order.  Results do
// not depend on which block runs an item.
//
// Block tile: 256 rows x 256 weight rows x 64 K, 256 threads = 4 waves in a
// 2 x 2 grid, each wave 128 x 128 as up to 4 x 4 MFMA 32x32x16 tiles with
// fp32 accumulators.  Operands go global -> LDS with the direct 16-byte LDS
// load of buffer instructions (no register staging), two stages,
// XOR-swizzled 16-byte chunks so MFMA fragment reads (32 rows, one K chunk)
// spread over the banks.  Row groups past the tile's row count are neither
// loaded nor multiplied: each wave runs a variant compiled for its number of
// live 32-row MFMA tiles (MT), so no accumulator is ever conditionally
// updated.
#include "common.h"

namespace moe {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x16_v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

namespace {

constexpr int P_TM = 256;          // rows per tile
constexpr int P_TN = 256;          // weight rows per tile
constexpr int P_TK = 64;           // K elements per stage
constexpr int P_ROWB = P_TK * 2;   // bytes per LDS row (128)
constexpr int P_STAGE = (P_TM + P_TN) * P_ROWB;  // 64 KB
constexpr int P_THREADS = 256;

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + expf(-a)); }

__device__ __forceinline__ int acc_row32(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// Buffer resource over [base, base + bytes): reads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// One direct 16-byte global -> LDS load per lane: lane l fills LDS bytes
// [l * 16, l * 16 + 16) of the 1 KB block at `lds`.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}

// Everything one wave needs to run a work item.
struct Item {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t a_off[8], b_off[8];  // byte offsets of this lane's 8 A and 8 B rows (swizzled chunk included)
  int a_groups;                 // 8-row groups of A that hold tile rows (wave-uniform)
  int wave, lane, lsw;
  int brow[4];                  // B rows of this wave's four 32-column MFMA tiles
  int mrow0;                    // first tile row of this wave
  int rows, row0, nk;
};

// Loads part Q (of 4) of the K slab starting at byte `kb` into stage buffer
// `dst`: instructions j = 2Q, 2Q+1 of the wave for A and for B.  Q = -1
// loads the whole slab.
template <int Q>
__device__ __forceinline__ void issue_part(const Item& it, uint8_t* __restrict__ dst, uint32_t kb) {
  uint8_t* sb = dst + P_TM * P_ROWB;
  constexpr int j0 = Q < 0 ? 0 : 2 * Q;
  constexpr int j1 = Q < 0 ? 8 : 2 * Q + 2;
#pragma unroll
  for (int j = j0; j < j1; ++j) {
    const int g = it.wave * 8 + j;
    if (g < it.a_groups) dma16(it.ra, dst + g * 1024, it.a_off[j], kb);
    dma16(it.rb, sb + g * 1024, it.b_off[j], kb);
  }
}
__device__ __forceinline__ void issue_stage(const Item& it, uint8_t* __restrict__ dst, uint32_t kb) {
  issue_part<-1>(it, dst, kb);
}

template <int MT>
__device__ __forceinline__ void load_frags(bf16x8_v (&af)[4], bf16x8_v (&bf)[4], const uint8_t* __restrict__ src,
                                           const Item& it, int kk) {
  const uint8_t* sb = src + P_TM * P_ROWB;
  const int c = kk * 2 + (it.lane >> 5);
  const int cofs = ((c ^ it.lsw) << 4);
  const int lr = it.lane & 31;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bf[j] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const uint4*>(sb + (it.brow[j] + lr) * P_ROWB + cofs));
#pragma unroll
  for (int i = 0; i < MT; ++i)
    af[i] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const uint4*>(src + (it.mrow0 + i * 32 + lr) * P_ROWB + cofs));
}

// One 64-wide K slab of MFMAs from stage buffer `src` (A rows, then B rows),
// with the loads of the next slab into `dst` spread over its four k-steps
// (a quarter before each k-step's MFMAs), so a wave never stalls behind a
// long burst of memory instructions.  Fragments are double-buffered by hand:
// the reads of k-step kk+1 are issued before the MFMAs of k-step kk, and a
// scheduling barrier after each k-step keeps the compiler from moving work
// across k-steps.  The stage pointers are restrict-qualified so the compiler
// knows the loads into one stage never alias the fragment reads of the other
// and does not wait for those loads before the MFMAs.
template <int MT, int KK>
__device__ __forceinline__ void kstep(f32x16_v (&acc)[MT > 0 ? MT : 1][4], bf16x8_v (&af)[2][4],
                                      bf16x8_v (&bf)[2][4], const Item& it, uint8_t* __restrict__ dst,
                                      const uint8_t* __restrict__ src, bool load_next, uint32_t next_kb) {
  if (load_next) issue_part<KK>(it, dst, next_kb);
  if constexpr (MT > 0) {
    if (KK + 1 < 4) load_frags<MT>(af[(KK + 1) & 1], bf[(KK + 1) & 1], src, it, KK + 1);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[KK & 1][i], bf[KK & 1][j], acc[i][j], 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int MT>
__device__ __forceinline__ void pipe_step(f32x16_v (&acc)[MT > 0 ? MT : 1][4], const Item& it,
                                          uint8_t* __restrict__ dst, const uint8_t* __restrict__ src,
                                          bool load_next, uint32_t next_kb) {
  bf16x8_v af[2][4], bf[2][4];
  if constexpr (MT > 0) load_frags<MT>(af[0], bf[0], src, it, 0);
  kstep<MT, 0>(acc, af, bf, it, dst, src, load_next, next_kb);
  kstep<MT, 1>(acc, af, bf, it, dst, src, load_next, next_kb);
  kstep<MT, 2>(acc, af, bf, it, dst, src, load_next, next_kb);
  kstep<MT, 3>(acc, af, bf, it, dst, src, load_next, next_kb);
}

__device__ __forceinline__ void store8(uint16_t* p, float4 a, float4 b) {
  uint4 q;
  q.x = pack_bf16x2(a.x, a.y);
  q.y = pack_bf16x2(a.z, a.w);
  q.z = pack_bf16x2(b.x, b.y);
  q.w = pack_bf16x2(b.z, b.w);
  *reinterpret_cast<uint4*>(p) = q;
}
__device__ __forceinline__ void store8(float* p, float4 a, float4 b) {
  *reinterpret_cast<float4*>(p) = a;
  *reinterpret_cast<float4*>(p + 4) = b;
}

// Epilogue.  Two passes of 128 rows (wave row 0, then 1): the waves of the
// pass write their fp32 accumulators to LDS (64 rows per stage buffer, one
// 1 KB row = 256 fp32), then all threads copy the rows out with 16-byte
// stores, applying SwiGLU (phase A: gate in columns 0..127, up in 128..255)
// and converting to the output type.  MT == 0: the wave has no rows.
template <bool PHASE_A, int MT, int MA, typename OT>
__device__ __forceinline__ void epilogue(const f32x16_v (&acc)[MA][4], const Item& it, uint8_t* st0, uint8_t* st1,
                                         int wm, int wn, int tid, OT* __restrict__ out, int Nd, int n) {
  constexpr int NC = PHASE_A ? P_TN / 2 : P_TN;  // output columns of the tile
  constexpr int LSTR = P_TN * 4;
  const int lcol = it.lane & 31;
  const long long col0 = (long long)n * NC;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
    if (wm == pass) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = i * 32 + acc_row32(e, it.lane);
          float* rowp = reinterpret_cast<float*>((r < 64 ? st0 : st1) + (r & 63) * LSTR);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int c = PHASE_A ? (j >> 1) * 128 + wn * 64 + (j & 1) * 32 + lcol : wn * 128 + j * 32 + lcol;
            rowp[c] = acc[i][j][e];
          }
        }
    }
    __syncthreads();
    constexpr int CH = NC / 8;                     // 8-value chunks per output row
    const int prow = it.rows - pass * 128;         // rows of this pass that exist
    const int nrow = prow < 0 ? 0 : (prow > 128 ? 128 : prow);
    for (int q = tid; q < nrow * CH; q += P_THREADS) {
      const int r = q / CH, ch = q % CH;
      const uint8_t* er = (r < 64 ? st0 : st1) + (r & 63) * LSTR;
      float4 v0 = *reinterpret_cast<const float4*>(er + ch * 32);
      float4 v1 = *reinterpret_cast<const float4*>(er + ch * 32 + 16);
      if (PHASE_A) {  // h = SiLU(gate) * up
        const float4 u0 = *reinterpret_cast<const float4*>(er + 512 + ch * 32);
        const float4 u1 = *reinterpret_cast<const float4*>(er + 512 + ch * 32 + 16);
        v0 = make_float4(silu_f(v0.x) * u0.x, silu_f(v0.y) * u0.y, silu_f(v0.z) * u0.z, silu_f(v0.w) * u0.w);
        v1 = make_float4(silu_f(v1.x) * u1.x, silu_f(v1.y) * u1.y, silu_f(v1.z) * u1.z, silu_f(v1.w) * u1.w);
      }
      OT* dst = out + (long long)(it.row0 + pass * 128 + r) * Nd + col0 + ch * 8;
      store8(dst, v0, v1);
    }
  }
}

// One work item for a wave with MT live 32-row MFMA tiles: accumulators,
// K loop (two-stage pipeline, unrolled by two so each step names its
// buffers) and epilogue, all in one instantiation.
template <bool PHASE_A, int MT, typename OT>
__device__ __forceinline__ void run_tile(const Item& it, uint8_t* st0, uint8_t* st1, int wm, int wn, int tid,
                                         OT* __restrict__ out, int Nd, int n) {
  constexpr int MA = MT > 0 ? MT : 1;
  f32x16_v acc[MA][4];
#pragma unroll
  for (int i = 0; i < MA; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // nk is even (K is a multiple of 128): the loop has a single exit.
  issue_stage(it, st0, 0);
  for (int s = 0; s < it.nk; s += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    pipe_step<MT>(acc, it, st1, st0, true, (uint32_t)(s + 1) * P_TK * 2u);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    pipe_step<MT>(acc, it, st0, st1, s + 2 < it.nk, (uint32_t)(s + 2) * P_TK * 2u);
  }
  epilogue<PHASE_A, MT, MA, OT>(acc, it, st0, st1, wm, wn, tid, out, Nd, n);
}

// PHASE_A: x = tokens [T, Kd] gathered by row_token, w = W13 [E, 2*Nd, Kd],
//          out = h [P, Nd] with SwiGLU; Nd = I, Kd = d.
// !PHASE_A: x = h [P, Kd], w = W2 [E, Nd, Kd], out = y [P, Nd]; Nd = d, Kd = I.
template <bool PHASE_A, typename OT>
__global__ __launch_bounds__(P_THREADS) void k_ffn_persistent(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ w,
                                                            const int32_t* __restrict__ row_token,
                                                            const int32_t* __restrict__ tile_map,
                                                            const int32_t* __restrict__ n_tiles, int Kd, int Nd,
                                                            int nt_total, uint32_t x_bytes,
                                                            int* __restrict__ counters, OT* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t st0[P_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[P_STAGE];
  __shared__ int s_item;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int xcd = blockIdx.x & 7;
  const int ntx = (nt_total - xcd + 7) >> 3;  // N tiles owned by this XCD
  const long long total = (long long)(*n_tiles) * ntx;
  const long long w_expert = (long long)(PHASE_A ? 2 : 1) * Nd * Kd;  // elements per expert

  for (;;) {
    __syncthreads();  // previous item done with LDS and s_item
    if (tid == 0) s_item = atomicAdd(&counters[xcd], 1);
    __syncthreads();
    const long long item = s_item;
    if (item >= total) break;
    const int tile = (int)(item / ntx);
    const int n = (int)(item % ntx) * 8 + xcd;
    const int4 tm = *reinterpret_cast<const int4*>(tile_map + 4LL * tile);
    const int seg = tm.x;

    // Operand streams: instruction j of a wave covers tile rows
    // 8 * (8 * wave + j) .. + 7 (lane l: row l / 8, physical chunk l & 7); the
    // lane fetches logical chunk c with physical = c ^ (row & 7) ^ ((row >> 3) & 1).
    Item it;
    it.rows = tm.z;
    it.row0 = tm.y;
    it.nk = Kd / P_TK;
    it.lane = lane;
    it.lsw = (lane & 7) ^ ((lane >> 3) & 1);
    it.wave = __builtin_amdgcn_readfirstlane(wave);
    it.a_groups = __builtin_amdgcn_readfirstlane((it.rows + 7) >> 3);
    it.rb = make_rsrc(w + (long long)seg * w_expert, (uint32_t)(w_expert * 2));
    it.ra = make_rsrc(x, x_bytes);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = (wave * 8 + j) * 8 + (lane >> 3);
      const uint32_t c16 = (uint32_t)((lane & 7) ^ (lane >> 3) ^ (j & 1)) * 16u;
      if (PHASE_A) {
        const int tok = r < it.rows ? row_token[it.row0 + r] : -1;
        // padding rows read past the end of the buffer, which yields zeros
        it.a_off[j] = tok >= 0 ? (uint32_t)tok * (uint32_t)Kd * 2u + c16 : 0x80000000u;
      } else {
        it.a_off[j] = r < it.rows ? (uint32_t)(it.row0 + r) * (uint32_t)Kd * 2u + c16 : 0x80000000u;
      }
      const int wrow = PHASE_A ? (r < 128 ? n * 128 + r : Nd + n * 128 + (r - 128)) : n * 256 + r;
      it.b_off[j] = (uint32_t)wrow * (uint32_t)Kd * 2u + c16;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      it.brow[j] = PHASE_A ? (j < 2 ? 0 : 128) + wn * 64 + (j & 1) * 32  // gate, gate, up, up
                           : wn * 128 + j * 32;
    it.mrow0 = wm * 128;
    int mt_live = (it.rows - it.mrow0 + 31) >> 5;  // 32-row MFMA tiles of this wave that hold rows
    mt_live = __builtin_amdgcn_readfirstlane(mt_live < 0 ? 0 : (mt_live > 4 ? 4 : mt_live));
    switch (mt_live) {
      case 4: run_tile<PHASE_A, 4, OT>(it, st0, st1, wm, wn, tid, out, Nd, n); break;
      case 3: run_tile<PHASE_A, 3, OT>(it, st0, st1, wm, wn, tid, out, Nd, n); break;
      case 2: run_tile<PHASE_A, 2, OT>(it, st0, st1, wm, wn, tid, out, Nd, n); break;
      case 1: run_tile<PHASE_A, 1, OT>(it, st0, st1, wm, wn, tid, out, Nd, n); break;
      default: run_tile<PHASE_A, 0, OT>(it, st0, st1, wm, wn, tid, out, Nd, n); break;
    }
  }
}

__global__ void k_zero_counters(int* c, int n) {
  if ((int)threadIdx.x < n) c[threadIdx.x] = 0;
}

int persistent_blocks() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!cached[dev]) {
    hipDeviceProp_t p;
    int cus = 256;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess && p.multiProcessorCount > 0) cus = p.multiProcessorCount;
    cached[dev] = (cus / 8) * 8 > 0 ? (cus / 8) * 8 : 8;
  }
  return cached[dev];
}

}  // namespace

bool ffn_bf16_persistent_ok(int d, int I) { return d % 256 == 0 && I % 128 == 0; }

// counters: 16 ints of device memory (8 per phase).
void launch_ffn_bf16_persistent(const uint16_t* x, const uint16_t* w13, const uint16_t* w2, const int32_t* row_token,
                                const int32_t* tile_map, const int32_t* n_tiles, int T, long long P, int d, int I,
                                uint16_t* h, void* y, bool y_f32, int* counters, hipStream_t st) {
  const int nb = persistent_blocks();
  const uint32_t x_bytes = (uint32_t)((long long)T * d * 2);
  const uint32_t h_bytes = (uint32_t)(P * I * 2);
  hipLaunchKernelGGL(k_zero_counters, dim3(1), dim3(64), 0, st, counters, 16);
  hipLaunchKernelGGL((k_ffn_persistent<true, uint16_t>), dim3(nb), dim3(P_THREADS), 0, st, x, w13, row_token,
                     tile_map, n_tiles, d, I, I / 128, x_bytes, counters, h);
  if (y_f32)
    hipLaunchKernelGGL((k_ffn_persistent<false, float>), dim3(nb), dim3(P_THREADS), 0, st, h, w2, row_token,
                       tile_map, n_tiles, I, d, d / 256, h_bytes, counters + 8, static_cast<float*>(y));
  else
    hipLaunchKernelGGL((k_ffn_persistent<false, uint16_t>), dim3(nb), dim3(P_THREADS), 0, st, h, w2, row_token,
                       tile_map, n_tiles, I, d, d / 256, h_bytes, counters + 8, static_cast<uint16_t*>(y));
}

}  // namespace moe
