// Persistent, XCD-aware grouped SwiGLU expert GEMMs on MFMA (gfx950): bf16,
// and E4M3 x E4M3 with tile / block scales.
//
// The expert FFNs of the combine equation in the "DeepSeek-V3 Technical
// Report" reading guide (xyznot.com, Method section 2), in the SwiGLU form
// this library uses: h = SiLU(x W_gate^T) * (x W_up^T), y = h W_down^T.  The
// FP8 variant follows the same page's "Key ideas" FP8 bullet: E4M3 operands,
// 1x128 activation tiles and 128x128 weight blocks, each with a scale.
//
// Work decomposition.  A work item is (row tile of the tile map, N tile).
// Phase A: N tile = 128 h columns = 128 gate rows + the 128 up rows of the
// same columns of W13.  Phase B: N tile = 256 columns of y (rows of W2).
// k_ffn_schedule deals whole experts to the 8 XCDs (largest first, snake
// order; a shared expert's tiles one by one), so an expert's weights are
// fetched by one XCD, and lists each XCD's items N-tile major, so the row
// tiles of an expert that share a weight slab run close together in that
// XCD's L2.  The kernel is persistent: 8 * (CUs / 8) blocks, block b runs on
// XCD b % 8 (workgroups are dealt to XCDs round robin) and pulls items from
// its XCD's list through an atomic counter, then helps the other XCDs.
// Results do not depend on which block runs an item.
//
// Block tile: 256 rows x 256 weight rows x 128 bytes of K per stage (64 bf16
// or 128 E4M3 values: one scale block), 256 threads = 4 waves in a 2 x 2
// grid, each wave 128 x 128 as up to 4 x 4 MFMA 32x32 tiles (bf16: 32x32x16;
// E4M3: the block-scaled 32x32x64, whose per-lane E8M0 scales carry the
// power-of-two tile and block scales, so scaling is exact and costs no extra
// work) with fp32 accumulators.  Operands go global -> LDS with the direct
// 16-byte LDS load of buffer instructions (no register staging), XOR-swizzled
// 16-byte chunks so MFMA fragment reads (32 rows, one K chunk) spread over
// the banks.  bf16: two A stages and three B stages, B loaded two stages
// ahead (deep_body); E4M3: two stages of A + its row scales and B (the row
// scales leave no room for a third B stage).  Rows past the tile's row count
// are loaded as zeros (out-of-range buffer loads fetch nothing) and 32-row
// MFMA tiles with no live row are not multiplied: each wave runs a variant
// compiled for its number of live tiles (MT), so no accumulator is ever
// conditionally updated.
#include "common.h"

namespace moe {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef int i32x8_v __attribute__((ext_vector_type(8)));
typedef float f32x16_v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

namespace {

constexpr int P_TM = 256;          // rows per tile
constexpr int P_TN = 256;          // weight rows per tile
constexpr int P_ROWB = 128;        // bytes of K per stage and row
constexpr int P_OPS = (P_TM + P_TN) * P_ROWB;  // A and B bytes of a stage (64 KB)
constexpr int P_THREADS = 256;

template <bool FP8>
struct Fmt {
  static constexpr int EB = FP8 ? 1 : 2;                 // bytes per element
  static constexpr int KSTEPS = FP8 ? 2 : 4;             // MFMA k-steps per stage
  static constexpr int STAGE = P_OPS + (FP8 ? 1024 : 0); // + 256 A-row scales (fp32)
};


__device__ __forceinline__ int acc_row32(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// E8M0 exponent byte of a power-of-two fp32 scale.
__device__ __forceinline__ int e8m0_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xFF); }

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
  __amdgpu_buffer_rsrc_t ra, rb, rs;  // A operand, B operand, A-row scales (FP8)
  uint32_t a_off[8], b_off[8];  // byte offsets of this lane's 8 A and 8 B rows (swizzled chunk included)
  uint32_t s_off;               // FP8: byte offset of the scale row of tile row 64 * wave + lane
  float bsc0, bsc1;             // FP8: lane l holds the B-block scale of K block l (gate / up, or the wave's block)
  int wave, lane, lsw;
  int brow[4];                  // B rows of this wave's four 32-column MFMA tiles
  int mrow0;                    // first tile row of this wave
  int rows, row0, nk;
  const int32_t* tok;           // fused combine: token of every permuted row
  const float* gate;            // fused combine: gate of every permuted row
};

// Loads part Q (of P) of the K slab starting at byte `kb` into stage buffer
// `dst`: A and B instructions j in [8Q/P, 8(Q+1)/P), plus (FP8, part 0) the
// A-row scales of the slab.  Q = -1 loads the whole slab.  `oob` is 0 or
// 0x80000000: the latter turns every load into an out-of-range one that only
// writes zeros to LDS, which lets the last step of a tile issue the same
// instructions as the others.  The K loop then has no branches, so the
// compiler cannot sink a step's MFMAs past the next barrier.  Row groups past
// the tile's rows carry out-of-range offsets for the same reason.
template <bool FP8, int Q, int P>
__device__ __forceinline__ void issue_part(const Item& it, uint8_t* __restrict__ dst, uint32_t kb, uint32_t oob) {
  uint8_t* sb = dst + P_TM * P_ROWB;
  constexpr int j0 = Q < 0 ? 0 : 8 * Q / P;
  constexpr int j1 = Q < 0 ? 8 : 8 * (Q + 1) / P;
#pragma unroll
  for (int j = j0; j < j1; ++j) {
    const int g = it.wave * 8 + j;
    dma16(it.ra, dst + g * 1024, it.a_off[j] | oob, kb);
    dma16(it.rb, sb + g * 1024, it.b_off[j] | oob, kb);
  }
  if constexpr (FP8) {
    if (Q <= 0)  // 4 bytes per lane: scale of tile row 64 * wave + lane for K block kb / 128
      __builtin_amdgcn_raw_ptr_buffer_load_lds(it.rs, (lds_void_t*)(dst + P_OPS + it.wave * 256), 4, it.s_off | oob,
                                               kb / P_ROWB * 4u, 0, 0);
  }
}

// E4M3 fragments: 32 bytes per lane (two 16-byte chunks of K step kk).  A and
// B use the same byte layout, and every scale is constant over the 64 K values
// of one MFMA, so the hardware's K order inside a lane does not matter.
__device__ __forceinline__ i32x8_v frag32(const uint8_t* row, int c0, int lsw) {
  const uint4 lo = *reinterpret_cast<const uint4*>(row + ((c0 ^ lsw) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(row + (((c0 + 1) ^ lsw) << 4));
  i32x8_v v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

template <int MT>
__device__ __forceinline__ void load_frags_fp8(i32x8_v (&af)[4], i32x8_v (&bf)[4], const uint8_t* __restrict__ src,
                                               const Item& it, int kk) {
  const uint8_t* sb = src + P_TM * P_ROWB;
  const int c0 = kk * 4 + (it.lane >> 5) * 2;
  const int lr = it.lane & 31;
#pragma unroll
  for (int j = 0; j < 4; ++j) bf[j] = frag32(sb + (it.brow[j] + lr) * P_ROWB, c0, it.lsw);
#pragma unroll
  for (int i = 0; i < MT; ++i) af[i] = frag32(src + (it.mrow0 + i * 32 + lr) * P_ROWB, c0, it.lsw);
}

// One stage of the E4M3 K loop (two k-steps of the block-scaled 32x32x64
// MFMA): half of the next slab's loads and the MFMAs of each k-step.
template <bool FP8, int MT>
__device__ __forceinline__ void pipe_step(f32x16_v (&acc)[MT > 0 ? MT : 1][4], const Item& it,
                                          uint8_t* __restrict__ dst, const uint8_t* __restrict__ src, int s,
                                          bool load_next, uint32_t next_kb) {
  static_assert(FP8, "the bf16 kernels use the deep K loop");
  // 32-byte E4M3 fragments are not double-buffered (register budget); an
  // FP8 k-step is long enough (16 MFMAs of 64 K) to cover the LDS reads.
  int sa[4] = {127, 127, 127, 127}, sbs[4] = {127, 127, 127, 127};
  if constexpr (MT > 0) {
    const float* scl = reinterpret_cast<const float*>(src + P_OPS);
#pragma unroll
    for (int i = 0; i < MT; ++i) sa[i] = e8m0_of(scl[it.mrow0 + i * 32 + (it.lane & 31)]);
    const int b0 = e8m0_of(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_uint(it.bsc0), s)));
    const int b1 = e8m0_of(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_uint(it.bsc1), s)));
    sbs[0] = b0; sbs[1] = b0; sbs[2] = b1; sbs[3] = b1;
  }
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    if (kk == 0)
      issue_part<true, 0, 2>(it, dst, next_kb, load_next ? 0u : 0x80000000u);
    else
      issue_part<true, 1, 2>(it, dst, next_kb, load_next ? 0u : 0x80000000u);
    if constexpr (MT > 0) {
      i32x8_v af[4], bf[4];
      load_frags_fp8<MT>(af, bf, src, it, kk);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0, sa[i], 0,
                                                                      sbs[j]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ------------------------------------------------------------------------
// bf16 K loop with three weight stages.  LDS holds two 32 KB stages of the
// activation tile (A) and three 32 KB stages of the weight tile (B): 160 KB.
// B is loaded two stages ahead and A one (deep_body), so the weight stream
// keeps 64 KB per CU in flight instead of 32 KB: a block is bound by its
// weight stream whenever its tile has few rows, and that rate is the bytes
// in flight over the memory latency.  Loads complete in issue order, so the
// wait before a stage's barrier names how many of the latest loads may still
// be outstanding (the B loads of two stages ahead).  Measured on the
// 8192-token prefill layer (expert GEMM call, identical outputs): 8.31 ms
// with the two-stage loop, 7.69 with three B stages, 7.44 with the next
// k-step's fragment reads interleaved one per MFMA, 7.21 with the barrier
// moved before the last k-step.
constexpr int D_AB = P_TM * P_ROWB;   // 32 KB: one stage of A or of B
constexpr int D_LDS = 5 * D_AB;       // A0 A1 B0 B1 B2

// Blocks [J0, J1) of the wave's 8 1 KB blocks of the A (or B) K slab at
// byte kb into dst.  oob as in issue_part.
template <int J0, int J1>
__device__ __forceinline__ void issue_a(const Item& it, uint8_t* __restrict__ dst, uint32_t kb, uint32_t oob) {
#pragma unroll
  for (int j = J0; j < J1; ++j) dma16(it.ra, dst + (it.wave * 8 + j) * 1024, it.a_off[j] | oob, kb);
}
template <int J0, int J1>
__device__ __forceinline__ void issue_b(const Item& it, uint8_t* __restrict__ dst, uint32_t kb, uint32_t oob) {
#pragma unroll
  for (int j = J0; j < J1; ++j) dma16(it.rb, dst + (it.wave * 8 + j) * 1024, it.b_off[j] | oob, kb);
}

template <int MT>
__device__ __forceinline__ void frags_ab(bf16x8_v (&af)[4], bf16x8_v (&bf)[4], const uint8_t* __restrict__ a_src,
                                         const uint8_t* __restrict__ b_src, const Item& it, int kk) {
  const int c = kk * 2 + (it.lane >> 5);
  const int cofs = ((c ^ it.lsw) << 4);
  const int lr = it.lane & 31;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bf[j] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const uint4*>(b_src + (it.brow[j] + lr) * P_ROWB + cofs));
#pragma unroll
  for (int i = 0; i < MT; ++i)
    af[i] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const uint4*>(a_src + (it.mrow0 + i * 32 + lr) * P_ROWB + cofs));
}

template <int MT>
__device__ __forceinline__ void mma_step(f32x16_v (&acc)[MT > 0 ? MT : 1][4], const bf16x8_v (&af)[4],
                                         const bf16x8_v (&bf)[4]) {
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
}

// s_waitcnt with vmcnt(8), expcnt and lgkmcnt left at their maxima (no wait).
constexpr unsigned WAIT_VM8 = (8u & 0xFu) | (0x7u << 4) | (0xFu << 8) | ((8u >> 4) << 14);
// vmcnt(8) and lgkmcnt(0); vmcnt(16) and lgkmcnt(0).
constexpr unsigned WAIT_VM8_LGKM0 = (8u & 0xFu) | (0x7u << 4) | ((8u >> 4) << 14);
constexpr unsigned WAIT_VM16_LGKM0 = (16u & 0xFu) | (0x7u << 4) | ((16u >> 4) << 14);

// Issue order inside a k-step: MFMA q, then LDS read q (the next k-step's
// fragments) and global load q, so the LDS serves the reads and the
// direct-to-LDS writes while the matrix pipe is busy.
template <int NMFMA, int NDS, int NVM>
__device__ __forceinline__ void order_kstep() {
  constexpr int N = NMFMA > NDS ? (NMFMA > NVM ? NMFMA : NVM) : (NDS > NVM ? NDS : NVM);
#pragma unroll
  for (int q = 0; q < N; ++q) {
    if (q < NMFMA) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (q < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (q < NVM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

// One stage s of the bf16 K loop.  On entry the fragments of k-step 0 are
// being read, A(s + 1) has been issued and B(s + 1) is in flight or landed.
//   k-step 0: MFMAs of k 0, fragments of k 1, B(s + 2) blocks 0-3 -> b_dst
//   k-step 1: MFMAs of k 1, fragments of k 2, B(s + 2) blocks 4-7
//   k-step 2: MFMAs of k 2, fragments of k 3
//   wait for this wave's LDS reads and for everything but B(s + 2), then the
//   barrier: A(s + 1) and B(s + 1) have landed for every wave, and no wave
//   reads A(s) or B(s) any more
//   k-step 3: MFMAs of k 3, fragments of k-step 0 of stage s + 1 (a_nxt,
//   b_nxt), A(s + 2) into the A(s) buffer (a_cur)
// So the reads that start a stage run under the last MFMAs of the one
// before, and B is loaded two stages ahead, A one.  The buffers named by
// different restrict pointers are distinct; A(s + 2) goes through a_cur
// itself, after the barrier.
template <int MT>
__device__ __forceinline__ void deep_body(f32x16_v (&acc)[MT > 0 ? MT : 1][4], bf16x8_v (&af)[2][4],
                                          bf16x8_v (&bf)[2][4], const Item& it, uint8_t* __restrict__ a_cur,
                                          const uint8_t* __restrict__ b_cur, const uint8_t* __restrict__ a_nxt,
                                          const uint8_t* __restrict__ b_nxt, uint8_t* __restrict__ b_dst,
                                          uint32_t b_kb, uint32_t b_oob, uint32_t a_kb, uint32_t a_oob) {
  constexpr int NM = 4 * MT, ND = MT > 0 ? MT + 4 : 0;
  issue_b<0, 4>(it, b_dst, b_kb, b_oob);
  if constexpr (MT > 0) {
    frags_ab<MT>(af[1], bf[1], a_cur, b_cur, it, 1);
    mma_step<MT>(acc, af[0], bf[0]);
  }
  order_kstep<NM, ND, 4>();
  __builtin_amdgcn_sched_barrier(0);
  issue_b<4, 8>(it, b_dst, b_kb, b_oob);
  if constexpr (MT > 0) {
    frags_ab<MT>(af[0], bf[0], a_cur, b_cur, it, 2);
    mma_step<MT>(acc, af[1], bf[1]);
  }
  order_kstep<NM, ND, 4>();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (MT > 0) {
    frags_ab<MT>(af[1], bf[1], a_cur, b_cur, it, 3);
    mma_step<MT>(acc, af[0], bf[0]);
  }
  order_kstep<NM, ND, 0>();
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(WAIT_VM8_LGKM0);  // own LDS reads done; A(s + 1), B(s + 1) landed
  __builtin_amdgcn_s_barrier();               // ... for every wave
  __builtin_amdgcn_sched_barrier(0);
  issue_a<0, 8>(it, a_cur, a_kb, a_oob);
  if constexpr (MT > 0) {
    frags_ab<MT>(af[0], bf[0], a_nxt, b_nxt, it, 0);
    mma_step<MT>(acc, af[1], bf[1]);
  }
  order_kstep<NM, ND, 8>();
  __builtin_amdgcn_sched_barrier(0);
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
__device__ __forceinline__ void store8(uint8_t*, float4, float4) {}  // E4M3 h is written by the quantising path

__device__ __forceinline__ float absmax8(float4 a, float4 b) {
  return fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
               fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
}

// A barrier for LDS traffic only: this wave's LDS accesses are complete,
// then every wave meets; global stores still in flight are not waited for
// (the fence of __syncthreads would wait for them).  The compiler moves no
// memory access across it.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Epilogue.  Phase B with bf16 output stores straight from the
// accumulators.  Otherwise two passes of 128 rows (wave row 0, then 1): the
// waves of the pass write their fp32 accumulators to LDS (64 rows per stage
// buffer, one 1 KB row = 256 fp32), then all threads copy the rows out with
// 16-byte stores, applying SwiGLU (phase A: gate in columns 0..127, up in
// 128..255) and converting to the output type.  With H_FP8 the 128 h values of a row
// are quantised as one 1x128 E4M3 tile (power-of-two scale, round to nearest
// even): the 16 threads holding a row find its amax with lane shuffles.
// MT == 0: the wave has no rows.
template <bool PHASE_A, bool H_FP8, int MT, int MA, typename OT, bool KEEP, bool FUSE = false>
__device__ __forceinline__ void epilogue(const f32x16_v (&acc)[MA][4], const Item& it, uint8_t* st0, uint8_t* st1,
                                         int wm, int wn, int tid, OT* __restrict__ out, float* __restrict__ out_scale,
                                         uint16_t* __restrict__ ab, uint16_t* __restrict__ hb, int Nd, int n) {
  constexpr int NC = PHASE_A ? P_TN / 2 : P_TN;  // output columns of the tile
  constexpr int LSTR = P_TN * 4;
  const int lcol = it.lane & 31;
  const long long col0 = (long long)n * NC;
  if constexpr (!PHASE_A && FUSE) {
    // Fused combine: out [T, Nd] fp32 holds the layer output; every token
    // row adds gate * y to its token's row with hardware fp32 atomics (one
    // 4-byte add per value; the 32 lanes of a row segment hit consecutive
    // columns).  The order of the adds is not fixed.
    static_assert(sizeof(OT) == 4, "the fused combine accumulates in fp32");
    float* ob = reinterpret_cast<float*>(out) + col0 + wn * 128 + lcol;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = wm * 128 + i * 32 + acc_row32(e, it.lane);
        if (r < it.rows) {
          const long long t = it.tok[it.row0 + r];
          const float g = it.gate[it.row0 + r];
          float* rowp = ob + t * Nd;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float v;
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(acc[i][j][e]));
            unsafeAtomicAdd(rowp + j * 32, g * v);
          }
        }
      }
    return;
  }
  if constexpr (!PHASE_A && sizeof(OT) == 2) {
    // bf16 y straight from the accumulators, one 2-byte store per value: no
    // LDS round trip and no barriers (6.4 -> 5.4 us per 256 x 256 item).
    // Each accumulator is read on its own; left to itself the compiler
    // copies all of them to VGPRs first and spills.
    uint16_t* ob = reinterpret_cast<uint16_t*>(out) + col0 + wn * 128 + lcol;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = wm * 128 + i * 32 + acc_row32(e, it.lane);
        if (r < it.rows) {
          uint16_t* rowp = ob + (long long)(it.row0 + r) * Nd;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float v;
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(acc[i][j][e]));
            rowp[j * 32] = f32_to_bf16(v);
          }
        }
      }
    return;
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    lds_sync();  // the K loop's (or the previous pass's) LDS reads are done
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
    lds_sync();
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
        if ((!H_FP8 || KEEP) && ab) {  // training: keep the pre-activations [a | b] for the backward pass
          uint16_t* abr = ab + (it.row0 + pass * 128 + r) * 2LL * Nd + col0 + ch * 8;
          store8(abr, v0, v1);
          store8(abr + Nd, u0, u1);
        }
        v0 = make_float4(silu(v0.x) * u0.x, silu(v0.y) * u0.y, silu(v0.z) * u0.z, silu(v0.w) * u0.w);
        v1 = make_float4(silu(v1.x) * u1.x, silu(v1.y) * u1.y, silu(v1.z) * u1.z, silu(v1.w) * u1.w);
      }
      const long long orow = it.row0 + pass * 128 + r;
      if constexpr (H_FP8) {
        float amax = absmax8(v0, v1);
#pragma unroll
        for (int o = 1; o < CH; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));  // the row's 16 threads
        const int k = pow2_scale_exp(amax);
        const float inv = exp2_int(-k);
        uint2 wv;
        wv.x = e4m3x4(v0.x * inv, v0.y * inv, v0.z * inv, v0.w * inv);
        wv.y = e4m3x4(v1.x * inv, v1.y * inv, v1.z * inv, v1.w * inv);
        uint8_t* dst = reinterpret_cast<uint8_t*>(out) + orow * Nd + col0 + ch * 8;
        *reinterpret_cast<uint2*>(dst) = wv;
        if (ch == 0) out_scale[orow * (Nd / 128) + n] = exp2_int(k);
        if (KEEP && hb) {  // training: h as phase B multiplies it, code x scale in bf16 (exact)
          const float sc = exp2_int(k);
          uint4 hv;
          hv.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv.x, sc, false));
          hv.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv.x, sc, true));
          hv.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv.y, sc, false));
          hv.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv.y, sc, true));
          *reinterpret_cast<uint4*>(hb + orow * Nd + col0 + ch * 8) = hv;
        }
      } else {
        store8(out + orow * Nd + col0 + ch * 8, v0, v1);
      }
    }
  }
}

// The successor of the current work item (k_ffn_persistent, phase B).
// Thread 0 claims index i of its XCD's list with an atomic add as the item
// starts; resolve() reads the list entry once the tile's K loop has waited
// for all its loads, before the epilogue issues its stores (read after
// them, the entry's load would also wait for the stores).  entry < 0: the
// list is drained.  Only wave 0's value is used.  Phase A claims as the
// tile ends: its items are long, and a claim one item ahead left blocks
// holding work at the end of the phase (bf16 call +2 %; phase B's claim
// ahead: E4M3 call -0.8 %, bf16 unchanged, in A/B runs).
struct NextItem {
  const int* list;
  int tot, i, entry;
  __device__ void resolve(int tid) {
    int e = -1;
    if (tid == 0 && i < tot) e = list[i];
    entry = __builtin_amdgcn_readfirstlane(e);
  }
};

// vmcnt(0) and lgkmcnt(0) as a builtin, so the compiler knows every load has
// completed; the empty asm statements keep memory accesses on their side.
__device__ __forceinline__ void wait_all_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x7u << 4);
  asm volatile("" ::: "memory");
}

// One work item for a wave with MT live 32-row MFMA tiles: accumulators,
// K loop (two-stage pipeline, unrolled by two so each step names its
// buffers and the loop has a single exit) and epilogue, all in one
// instantiation.
template <bool FP8, bool PHASE_A, int MT, typename OT, bool KEEP, bool FUSE>
__device__ __forceinline__ void run_tile(const Item& it, uint8_t* st0, uint8_t* st1, int wm, int wn, int tid,
                                         OT* __restrict__ out, float* __restrict__ out_scale,
                                         uint16_t* __restrict__ ab, uint16_t* __restrict__ hb, int Nd, int n,
                                         NextItem& nx) {
  constexpr int MA = MT > 0 ? MT : 1;
  f32x16_v acc[MA][4];
#pragma unroll
  for (int i = 0; i < MA; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  issue_part<FP8, -1, 1>(it, st0, 0, 0u);
  for (int s = 0; s < it.nk; s += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    pipe_step<FP8, MT>(acc, it, st1, st0, s, true, (uint32_t)(s + 1) * P_ROWB);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    pipe_step<FP8, MT>(acc, it, st0, st1, s + 1, s + 2 < it.nk, (uint32_t)(s + 2) * P_ROWB);
  }
  wait_all_loads();  // the last step's zero loads land before LDS is reused
  if constexpr (!PHASE_A) nx.resolve(tid);  // (see NextItem)
  epilogue<PHASE_A, FP8 && PHASE_A, MT, MA, OT, KEEP, FUSE>(acc, it, st0, st1, wm, wn, tid, out, out_scale, ab, hb, Nd,
                                                      n);
}

// run_tile of the bf16 kernels: the K loop of deep_body (two A stages,
// three B stages, rotated each stage), then the epilogue.  lds = D_LDS
// bytes; the epilogue stages its rows through the first 128 KB.
template <bool PHASE_A, int MT, typename OT, bool KEEP, bool FUSE>
__device__ __forceinline__ void run_tile_deep(const Item& it, uint8_t* lds, int wm, int wn, int tid,
                                              OT* __restrict__ out, uint16_t* __restrict__ ab, int Nd, int n,
                                              NextItem& nx) {
  constexpr int MA = MT > 0 ? MT : 1;
  f32x16_v acc[MA][4];
#pragma unroll
  for (int i = 0; i < MA; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  uint8_t* a0 = lds;
  uint8_t* a1 = lds + D_AB;
  uint8_t* b0 = lds + 2 * D_AB;
  uint8_t* b1 = lds + 3 * D_AB;
  uint8_t* b2 = lds + 4 * D_AB;
  const uint32_t OOB = 0x80000000u;
  // prologue: A(0), B(0), then B(1), A(1) (all buffers are free); wait for
  // the first two, read the fragments of stage 0, k-step 0
  issue_a<0, 8>(it, a0, 0, 0u);
  issue_b<0, 8>(it, b0, 0, 0u);
  issue_b<0, 8>(it, b1, P_ROWB, it.nk > 1 ? 0u : OOB);
  issue_a<0, 8>(it, a1, P_ROWB, it.nk > 1 ? 0u : OOB);
  __builtin_amdgcn_s_waitcnt(WAIT_VM16_LGKM0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  bf16x8_v af[2][4], bf[2][4];
  if constexpr (MT > 0) frags_ab<MT>(af[0], bf[0], a0, b0, it, 0);
  for (int s = 0; s < it.nk; ++s) {
    deep_body<MT>(acc, af, bf, it, a0, b0, a1, b1, b2, (uint32_t)(s + 2) * P_ROWB, s + 2 < it.nk ? 0u : OOB,
                  (uint32_t)(s + 2) * P_ROWB, s + 2 < it.nk ? 0u : OOB);
    uint8_t* t = a0; a0 = a1; a1 = t;
    t = b0; b0 = b1; b1 = b2; b2 = t;
  }
  wait_all_loads();  // the last zero loads land before LDS is reused
  if constexpr (!PHASE_A) nx.resolve(tid);  // (see NextItem)
  epilogue<PHASE_A, false, MT, MA, OT, KEEP, FUSE>(acc, it, lds, lds + 2 * D_AB, wm, wn, tid, out, nullptr, ab, nullptr,
                                             Nd, n);
}

// ------------------------------------------------------------------------
// LDS of the kernel.  E4M3: two stages of A + row scales and B as separate
// arrays (the compiler then knows they never overlap), and the item word.
// bf16: the D_LDS bytes of the deep K loop; the item word sits in the third
// B stage, which neither the prologue's loads nor the epilogue touch: it is
// first written by the loads of stage 0's body, issued after the prologue's
// barrier, when every wave has read the word.
template <bool FP8>
struct KernelLds;
template <>
struct KernelLds<true> {
  __attribute__((aligned(1024))) uint8_t st0[Fmt<true>::STAGE];
  __attribute__((aligned(1024))) uint8_t st1[Fmt<true>::STAGE];
  int item_word;
  __device__ uint8_t* base() { return st0; }
  __device__ uint8_t* stage0() { return st0; }
  __device__ uint8_t* stage1() { return st1; }
  __device__ int* item() { return &item_word; }
};
template <>
struct KernelLds<false> {
  __attribute__((aligned(1024))) uint8_t lds[D_LDS];
  __device__ uint8_t* base() { return lds; }
  __device__ uint8_t* stage0() { return lds; }
  __device__ uint8_t* stage1() { return lds + 2 * D_AB; }
  __device__ int* item() { return reinterpret_cast<int*>(lds + 4 * D_AB); }
};

// PHASE_A: x = tokens [T, Kd] gathered by row_token, w = W13 [E, 2*Nd, Kd],
//          out = h [P, Nd] with SwiGLU; Nd = I, Kd = d.
// !PHASE_A: x = h [P, Kd], w = W2 [E, Nd, Kd], out = y [P, Nd]; Nd = d, Kd = I.
// FP8: x, w are E4M3 codes; x_scale [rows of x, Kd/128] and
//      w_scale [E, rows of w / 128, Kd/128] are power-of-two fp32 scales;
//      phase A writes h as E4M3 codes with scales out_scale [P, Nd/128].
// ab (bf16 phase A only, may be NULL): [P, 2 Nd] gets the pre-activations
//      a (columns 0..Nd-1) and b (Nd..2Nd-1) of every token row.
// FUSE (phase B): out = the layer output [T, Nd] fp32; each token row adds
//      row_gate[row] * y to the row of its token (fused combine).
template <bool FP8, bool PHASE_A, typename OT, bool KEEP = false, bool FUSE = false>
__global__ __launch_bounds__(P_THREADS) void k_ffn_persistent(const uint8_t* __restrict__ x,
                                                            const uint8_t* __restrict__ w,
                                                            const float* __restrict__ x_scale,
                                                            const float* __restrict__ w_scale,
                                                            const int32_t* __restrict__ row_token,
                                                            const int32_t* __restrict__ tile_map,
                                                            const int32_t* __restrict__ n_tiles, int Kd, int Nd,
                                                            uint32_t x_bytes, uint32_t xs_bytes,
                                                            int* __restrict__ counters,
                                                            const int* __restrict__ totals,
                                                            const int* __restrict__ offsets,
                                                            const int* __restrict__ items,
                                                            OT* __restrict__ out, float* __restrict__ out_scale,
                                                            uint16_t* __restrict__ ab,
                                                            uint16_t* __restrict__ hb,
                                                            const float* __restrict__ row_gate) {
  constexpr int EB = Fmt<FP8>::EB;
  __shared__ KernelLds<FP8> L;
  uint8_t* lds = L.base();
  uint8_t* st0 = L.stage0();
  uint8_t* st1 = L.stage1();
  int* s_item_p = L.item();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int xcd = blockIdx.x & 7;
  const int wrows = PHASE_A ? 2 * Nd : Nd;     // weight rows per expert
  const long long w_expert = (long long)wrows * Kd * EB;  // bytes per expert
  const int kblocks = Kd * EB / P_ROWB;        // K blocks (stages) of a row

  // Items are claimed by thread 0 and passed on through the LDS item word.
  // In phase B the claim of an item's successor on this XCD's list (an
  // atomic add) is issued when the item starts and its result read after
  // the K loop (NextItem); phase A claims as the tile ends.  When the list
  // is drained, the other XCDs' lists are searched as the tile ends.  The
  // barriers between items wait for LDS traffic only: the epilogue's global
  // stores drain under the next item's set-up (a __syncthreads fence would
  // wait for them).
  const int tot_x = totals[xcd], off_x = offsets[xcd];
  auto steal = [&](int k0) {
    int got = -1;
    for (int k = k0; k < 8 && got < 0; ++k) {
      const int y = (xcd + k) & 7;
      const int tot = totals[y];
      if (__atomic_load_n(&counters[y], __ATOMIC_RELAXED) >= tot) continue;
      const int i = atomicAdd(&counters[y], 1);
      if (i < tot) got = items[offsets[y] + i];
    }
    return got;
  };
  if (tid == 0) *s_item_p = steal(0);
  lds_sync();
  int entry = *s_item_p;
  constexpr bool EARLY = !PHASE_A;  // see NextItem
  while (entry >= 0) {
    NextItem nx{items + off_x, tot_x, 0, -1};
    if (EARLY && tid == 0) nx.i = atomicAdd(&counters[xcd], 1);
    const int tile = entry >> 8;
    const int n = entry & 255;
    const int4 tm = *reinterpret_cast<const int4*>(tile_map + 4LL * tile);
    const int seg = tm.x;

    // Operand streams: instruction j of a wave covers tile rows
    // 8 * (8 * wave + j) .. + 7 (lane l: row l / 8, physical chunk l & 7); the
    // lane fetches logical chunk c with physical = c ^ (row & 7) ^ ((row >> 3) & 1).
    Item it;
    it.rows = tm.w;  // token rows; the tile's padding rows are skipped
    it.row0 = tm.y;
    it.nk = kblocks;
    it.tok = row_token;
    it.gate = row_gate;
    it.lane = lane;
    it.lsw = (lane & 7) ^ ((lane >> 3) & 1);
    it.wave = __builtin_amdgcn_readfirstlane(wave);
    it.rb = make_rsrc(w + seg * w_expert, (uint32_t)w_expert);
    it.ra = make_rsrc(x, x_bytes);
    const uint32_t row_bytes = (uint32_t)Kd * EB;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = (wave * 8 + j) * 8 + (lane >> 3);
      const uint32_t c16 = (uint32_t)((lane & 7) ^ (lane >> 3) ^ (j & 1)) * 16u;
      if (PHASE_A) {
        const int tok = r < it.rows ? row_token[it.row0 + r] : -1;
        // padding rows read past the end of the buffer, which yields zeros
        it.a_off[j] = tok >= 0 ? (uint32_t)tok * row_bytes + c16 : 0x80000000u;
      } else {
        it.a_off[j] = r < it.rows ? (uint32_t)(it.row0 + r) * row_bytes + c16 : 0x80000000u;
      }
      const int wrow = PHASE_A ? (r < 128 ? n * 128 + r : Nd + n * 128 + (r - 128)) : n * 256 + r;
      it.b_off[j] = (uint32_t)wrow * row_bytes + c16;
    }
    if constexpr (FP8) {
      it.rs = make_rsrc(x_scale, xs_bytes);
      const int r = wave * 64 + lane;  // scale row streamed by this lane
      int srow = -1;
      if (PHASE_A)
        srow = r < it.rows ? row_token[it.row0 + r] : -1;
      else
        srow = r < it.rows ? it.row0 + r : -1;
      it.s_off = srow >= 0 ? (uint32_t)srow * (uint32_t)kblocks * 4u : 0x80000000u;
      // B-block scales of this wave's columns, one K block per lane (kblocks <= 64)
      const float* ws = w_scale + (long long)seg * (wrows / 128) * kblocks;
      const int blk0 = PHASE_A ? n : 2 * n + wn;
      const int blk1 = PHASE_A ? Nd / 128 + n : blk0;
      it.bsc0 = lane < kblocks ? ws[(long long)blk0 * kblocks + lane] : 1.0f;
      it.bsc1 = lane < kblocks ? ws[(long long)blk1 * kblocks + lane] : 1.0f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      it.brow[j] = PHASE_A ? (j < 2 ? 0 : 128) + wn * 64 + (j & 1) * 32  // gate, gate, up, up
                           : wn * 128 + j * 32;
    it.mrow0 = wm * 128;
    int mt_live = (it.rows - it.mrow0 + 31) >> 5;  // 32-row MFMA tiles of this wave that hold rows
    mt_live = __builtin_amdgcn_readfirstlane(mt_live < 0 ? 0 : (mt_live > 4 ? 4 : mt_live));
    if constexpr (FP8) {
      switch (mt_live) {
        case 4: run_tile<FP8, PHASE_A, 4, OT, KEEP, FUSE>(it, st0, st1, wm, wn, tid, out, out_scale, ab, hb, Nd, n, nx); break;
        case 3: run_tile<FP8, PHASE_A, 3, OT, KEEP, FUSE>(it, st0, st1, wm, wn, tid, out, out_scale, ab, hb, Nd, n, nx); break;
        case 2: run_tile<FP8, PHASE_A, 2, OT, KEEP, FUSE>(it, st0, st1, wm, wn, tid, out, out_scale, ab, hb, Nd, n, nx); break;
        case 1: run_tile<FP8, PHASE_A, 1, OT, KEEP, FUSE>(it, st0, st1, wm, wn, tid, out, out_scale, ab, hb, Nd, n, nx); break;
        default: run_tile<FP8, PHASE_A, 0, OT, KEEP, FUSE>(it, st0, st1, wm, wn, tid, out, out_scale, ab, hb, Nd, n, nx); break;
      }
    } else {
      switch (mt_live) {
        case 4: run_tile_deep<PHASE_A, 4, OT, KEEP, FUSE>(it, lds, wm, wn, tid, out, ab, Nd, n, nx); break;
        case 3: run_tile_deep<PHASE_A, 3, OT, KEEP, FUSE>(it, lds, wm, wn, tid, out, ab, Nd, n, nx); break;
        case 2: run_tile_deep<PHASE_A, 2, OT, KEEP, FUSE>(it, lds, wm, wn, tid, out, ab, Nd, n, nx); break;
        case 1: run_tile_deep<PHASE_A, 1, OT, KEEP, FUSE>(it, lds, wm, wn, tid, out, ab, Nd, n, nx); break;
        default: run_tile_deep<PHASE_A, 0, OT, KEEP, FUSE>(it, lds, wm, wn, tid, out, ab, Nd, n, nx); break;
      }
    }
    lds_sync();  // every wave done with LDS and the item word
    if (tid == 0) *s_item_p = EARLY && nx.entry >= 0 ? nx.entry : steal(EARLY ? 1 : 0);
    lds_sync();
    entry = *s_item_p;
  }
}

// Work lists of the two GEMM phases (one block of 1024 threads).
//
// A unit is a routed expert (all its tiles) or one tile of a shared expert.
// Units are dealt to the 8 XCDs largest first in snake order, so an expert's
// weights and its row tiles meet in one L2 while the work stays balanced;
// the big shared segments spread over all XCDs.
// Within a unit the items run N-tile major (all row tiles of the unit for N
// tile 0, then 1, ...), so concurrent blocks of an XCD share weight slabs.
// An item is (tile << 8) | N tile.
//
// sched: [0, 16) work counters (phase A 0..7, B 8..15), [16, 24) / [24, 32)
// items per XCD, [32, 40) / [40, 48) first item of each XCD, then the item
// lists of phase A (cap * ntA) and B (cap * ntB).
constexpr int SCHED_HDR = 64;
constexpr int SCHED_A_MODE = 1;
constexpr int SCHED_SMALL = 128;
constexpr int SCHED_MAXU = 4096;

__global__ __launch_bounds__(1024) void k_ffn_schedule(const int32_t* __restrict__ tile_map,
                                                       const int32_t* __restrict__ n_tiles, int Nr, int ntA,
                                                       int ntB, int cap, int* __restrict__ sched) {
  __shared__ int s_seg[SCHED_MAXU], s_trows[SCHED_MAXU];
  __shared__ int s_ustart[SCHED_MAXU + 1], s_urows[SCHED_MAXU], s_order[SCHED_MAXU];
  __shared__ int s_uoffA[SCHED_MAXU], s_uoffB[SCHED_MAXU];
  __shared__ unsigned char s_uxcd[SCHED_MAXU];
  __shared__ int s_xlist[SCHED_MAXU + 16];  // each XCD's units in deal order
  __shared__ int s_part[1024];
  __shared__ int s_nu, s_xA[8], s_xB[8];
  const int tid = threadIdx.x;
  const int tiles = min(*n_tiles, min(cap, SCHED_MAXU));
  if (tid < 16) sched[tid] = 0;
  for (int t = tid; t < tiles; t += 1024) {
    const int4 tm = *reinterpret_cast<const int4*>(tile_map + 4LL * t);
    s_seg[t] = tm.x;
    s_trows[t] = tm.w;
  }
  __syncthreads();
  // unit starts, numbered by a scan (4 tiles per thread)
  int flags[4], cnt = 0;
  for (int j = 0; j < 4; ++j) {
    const int t = tid * 4 + j;
    flags[j] = t < tiles && (t == 0 || s_seg[t] != s_seg[t - 1] || s_seg[t] >= Nr);
    cnt += flags[j];
  }
  s_part[tid] = cnt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? s_part[tid - o] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int u = s_part[tid] - cnt - 1;
  for (int j = 0; j < 4; ++j) {
    const int t = tid * 4 + j;
    if (t < tiles) {
      u += flags[j];
      if (flags[j]) s_ustart[u] = t;
    }
  }
  if (tid == 1023) s_nu = s_part[1023];
  __syncthreads();
  const int nu = s_nu;
  if (tid == 0) s_ustart[nu] = tiles;
  __syncthreads();
  for (int v = tid; v < nu; v += 1024) {
    int rows = 0;
    for (int t = s_ustart[v]; t < s_ustart[v + 1]; ++t) rows += s_trows[t];
    s_urows[v] = rows;
  }
  __syncthreads();
  // largest units first (ties: lower index first); plain rank by counting
  for (int v = tid; v < nu; v += 1024) {
    int rank = 0;
    if (nu <= 1024) {
      const int rv = s_urows[v];
      for (int w = 0; w < nu; ++w) rank += (s_urows[w] > rv) || (s_urows[w] == rv && w < v);
    } else {
      rank = v;  // many units: keep tile-map order
    }
    s_order[rank] = v;
  }
  __syncthreads();
  // Deal the units in rank order in snake rounds (0..7, 7..0, ...), each
  // round's largest to the XCD that got the smallest of the last round.  Then
  // one thread per XCD walks its units to place their items: phase A largest
  // unit first; phase B alternately from the large and the small end, so the
  // weight-streaming items of few-row experts run next to the MFMA-bound
  // items of many-row ones.
  if (tid < 8) {
    const int x = tid;
    const int stride = (nu + 7) / 8 + 1;  // an XCD gets at most one unit per round of 8
    int nA = 0, m = 0;
    for (int i = 0;; ++i) {
      const int r = 8 * i + ((i & 1) ? 7 - x : x);
      if (r >= nu) break;
      const int v = s_order[r];
      const int len = s_ustart[v + 1] - s_ustart[v];
      s_uxcd[v] = (unsigned char)x;
      nA += len * ntA;
      s_xlist[x * stride + m++] = v;
    }
    {
      // phase A order (SCHED_A_MODE): 0 largest first; 1 alternately from
      // both ends; 2 units of at most SCHED_SMALL rows merged into the
      // larger ones so that their items stay evenly spread over the list
      int oA = 0;
      if (SCHED_A_MODE == 0) {
        for (int k = 0; k < m; ++k) {
          const int v = s_xlist[x * stride + k];
          s_uoffA[v] = oA;
          oA += (s_ustart[v + 1] - s_ustart[v]) * ntA;
        }
      } else if (SCHED_A_MODE == 1) {
        for (int k = 0; k < m; ++k) {
          const int v = s_xlist[x * stride + ((k & 1) ? m - 1 - (k >> 1) : (k >> 1))];
          s_uoffA[v] = oA;
          oA += (s_ustart[v + 1] - s_ustart[v]) * ntA;
        }
      } else {
        int ks = m;
        while (ks > 0 && s_urows[s_xlist[x * stride + ks - 1]] <= SCHED_SMALL) --ks;
        long long TL = 0, TS = 0, cL = 0, cS = 0;
        for (int k = 0; k < m; ++k) {
          const long long it = s_ustart[s_xlist[x * stride + k] + 1] - s_ustart[s_xlist[x * stride + k]];
          if (k < ks) TL += it; else TS += it;
        }
        int i = 0, j = ks;
        while (i < ks || j < m) {
          const bool small = j < m && (i >= ks || cS * TL < cL * TS);
          const int v = s_xlist[x * stride + (small ? j++ : i++)];
          const int len = s_ustart[v + 1] - s_ustart[v];
          s_uoffA[v] = oA;
          oA += len * ntA;
          if (small) cS += len; else cL += len;
        }
      }
    }
    int nB = 0;
    for (int k = 0; k < m; ++k) {
      const int v = s_xlist[x * stride + ((k & 1) ? m - 1 - (k >> 1) : (k >> 1))];
      s_uoffB[v] = nB;
      nB += (s_ustart[v + 1] - s_ustart[v]) * ntB;
    }
    s_xA[x] = nA;
    s_xB[x] = nB;
  }
  __syncthreads();
  if (tid == 0) {
    int oa = 0, ob = 0;
    for (int x = 0; x < 8; ++x) {
      const int na = s_xA[x], nb = s_xB[x];
      sched[16 + x] = na;
      sched[24 + x] = nb;
      sched[32 + x] = oa;
      sched[40 + x] = ob;
      s_xA[x] = oa;
      s_xB[x] = ob;
      oa += na;
      ob += nb;
    }
  }
  __syncthreads();
  int* listA = sched + SCHED_HDR;
  int* listB = listA + (long long)cap * ntA;
  // one thread per (unit, N tile): the unit's row tiles for that N tile
  for (int q = tid; q < nu * ntA; q += 1024) {
    const int v = q / ntA, n = q - v * ntA;
    const int t0 = s_ustart[v], len = s_ustart[v + 1] - t0;
    int* la = listA + s_xA[s_uxcd[v]] + s_uoffA[v] + n * len;
    for (int j = 0; j < len; ++j) la[j] = ((t0 + j) << 8) | n;
  }
  for (int q = tid; q < nu * ntB; q += 1024) {
    const int v = q / ntB, n = q - v * ntB;
    const int t0 = s_ustart[v], len = s_ustart[v + 1] - t0;
    int* lb = listB + s_xB[s_uxcd[v]] + s_uoffB[v] + n * len;
    for (int j = 0; j < len; ++j) lb[j] = ((t0 + j) << 8) | n;
  }
}

// One block per CU, a multiple of 8 so every XCD gets the same count (the
// CU count is queried on every call: no state is kept between calls).
int persistent_blocks() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return (cus / 8) * 8 > 0 ? (cus / 8) * 8 : 8;
}

}  // namespace

bool ffn_bf16_persistent_ok(int d, int I) { return d % 256 == 0 && I % 128 == 0 && I / 128 <= 255 && d / 256 <= 255; }
bool ffn_fp8_persistent_ok(int d, int I) { return d % 256 == 0 && I % 256 == 0 && d / 128 <= 64 && I / 128 <= 64; }

size_t ffn_schedule_bytes(long long tiles_cap, int ntA, int ntB) {
  const size_t b = 4 * ((size_t)SCHED_HDR + (size_t)tiles_cap * (ntA + ntB));
  return (b + 255) / 256 * 256;
}
int ffn_schedule_max_tiles() { return SCHED_MAXU; }

namespace {

struct PhaseSched {
  int* cnt;
  const int* tot;
  const int* off;
  const int* items;
};

PhaseSched phase_sched(int* sched, int phase, int cap, int ntA) {
  PhaseSched p;
  p.cnt = sched + 8 * phase;
  p.tot = sched + 16 + 8 * phase;
  p.off = sched + 32 + 8 * phase;
  p.items = sched + SCHED_HDR + (phase ? (long long)cap * ntA : 0);
  return p;
}

}  // namespace

// sched: ffn_schedule_bytes(cap, I / 128, d / 256) bytes of device memory;
// cap >= the tile count (at most ffn_schedule_max_tiles()).
void launch_ffn_bf16_persistent(const uint16_t* x, const uint16_t* w13, const uint16_t* w2, const int32_t* row_token,
                                const int32_t* tile_map, const int32_t* n_tiles, int T, long long P, int d, int I,
                                int Nr, int cap, uint16_t* h, uint16_t* ab, void* y, bool y_f32, int* sched,
                                hipStream_t st, const float* row_gate) {
  const int nb = persistent_blocks();
  const uint32_t x_bytes = (uint32_t)((long long)T * d * 2);
  const uint32_t h_bytes = (uint32_t)(P * I * 2);
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
  const int ntA = I / 128, ntB = d / 256;
  hipLaunchKernelGGL(k_ffn_schedule, dim3(1), dim3(1024), 0, st, tile_map, n_tiles, Nr, ntA, ntB, cap, sched);
  const PhaseSched a = phase_sched(sched, 0, cap, ntA), b = phase_sched(sched, 1, cap, ntA);
  hipLaunchKernelGGL((k_ffn_persistent<false, true, uint16_t>), dim3(nb), dim3(P_THREADS), 0, st, xb,
                     reinterpret_cast<const uint8_t*>(w13), nullptr, nullptr, row_token, tile_map, n_tiles, d, I,
                     x_bytes, 0u, a.cnt, a.tot, a.off, a.items, h, nullptr, ab, nullptr, nullptr);
  const uint8_t* hb = reinterpret_cast<const uint8_t*>(h);
  if (row_gate)  // fused combine: y is the layer output [T, d] fp32
    hipLaunchKernelGGL((k_ffn_persistent<false, false, float, false, true>), dim3(nb), dim3(P_THREADS), 0, st, hb,
                       reinterpret_cast<const uint8_t*>(w2), nullptr, nullptr, row_token, tile_map, n_tiles, I, d,
                       h_bytes, 0u, b.cnt, b.tot, b.off, b.items, static_cast<float*>(y), nullptr, nullptr, nullptr,
                       row_gate);
  else if (y_f32)
    hipLaunchKernelGGL((k_ffn_persistent<false, false, float>), dim3(nb), dim3(P_THREADS), 0, st, hb,
                       reinterpret_cast<const uint8_t*>(w2), nullptr, nullptr, row_token, tile_map, n_tiles, I, d,
                       h_bytes, 0u, b.cnt, b.tot, b.off, b.items, static_cast<float*>(y), nullptr, nullptr, nullptr,
                       nullptr);
  else
    hipLaunchKernelGGL((k_ffn_persistent<false, false, uint16_t>), dim3(nb), dim3(P_THREADS), 0, st, hb,
                       reinterpret_cast<const uint8_t*>(w2), nullptr, nullptr, row_token, tile_map, n_tiles, I, d,
                       h_bytes, 0u, b.cnt, b.tot, b.off, b.items, static_cast<uint16_t*>(y), nullptr, nullptr,
                       nullptr, nullptr);
}

// E4M3 x E4M3: x codes [T, d] with x_scale [T, d/128]; W13 / W2 codes with
// block scales; h (workspace) = codes [P, I] then scales [P, I/128].
// Training (ab, hb not NULL): phase A also writes [a | b] [P, 2I] and h
// [P, I] (its E4M3 value) in bf16.
void launch_ffn_fp8_persistent(const uint8_t* x, const float* x_scale, const uint8_t* w13, const float* w13_scale,
                               const uint8_t* w2, const float* w2_scale, const int32_t* row_token,
                               const int32_t* tile_map, const int32_t* n_tiles, int T, long long P, int d, int I,
                               int Nr, int cap, uint8_t* h, float* h_scale, void* y, bool y_f32, int* sched,
                               hipStream_t st, uint16_t* ab, uint16_t* hb, const float* row_gate) {
  const int nb = persistent_blocks();
  const uint32_t x_bytes = (uint32_t)((long long)T * d);
  const uint32_t xs_bytes = (uint32_t)((long long)T * (d / 128) * 4);
  const uint32_t h_bytes = (uint32_t)(P * I);
  const uint32_t hs_bytes = (uint32_t)(P * (I / 128) * 4);
  const int ntA = I / 128, ntB = d / 256;
  hipLaunchKernelGGL(k_ffn_schedule, dim3(1), dim3(1024), 0, st, tile_map, n_tiles, Nr, ntA, ntB, cap, sched);
  const PhaseSched a = phase_sched(sched, 0, cap, ntA), b = phase_sched(sched, 1, cap, ntA);
  if (ab || hb)
    hipLaunchKernelGGL((k_ffn_persistent<true, true, uint8_t, true>), dim3(nb), dim3(P_THREADS), 0, st, x, w13,
                       x_scale, w13_scale, row_token, tile_map, n_tiles, d, I, x_bytes, xs_bytes, a.cnt, a.tot, a.off,
                       a.items, h, h_scale, ab, hb, nullptr);
  else
    hipLaunchKernelGGL((k_ffn_persistent<true, true, uint8_t>), dim3(nb), dim3(P_THREADS), 0, st, x, w13, x_scale,
                       w13_scale, row_token, tile_map, n_tiles, d, I, x_bytes, xs_bytes, a.cnt, a.tot, a.off, a.items,
                       h, h_scale, nullptr, nullptr, nullptr);
  if (row_gate)  // fused combine: y is the layer output [T, d] fp32
    hipLaunchKernelGGL((k_ffn_persistent<true, false, float, false, true>), dim3(nb), dim3(P_THREADS), 0, st, h, w2,
                       h_scale, w2_scale, row_token, tile_map, n_tiles, I, d, h_bytes, hs_bytes, b.cnt, b.tot, b.off,
                       b.items, static_cast<float*>(y), nullptr, nullptr, nullptr, row_gate);
  else if (y_f32)
    hipLaunchKernelGGL((k_ffn_persistent<true, false, float>), dim3(nb), dim3(P_THREADS), 0, st, h, w2, h_scale,
                       w2_scale, row_token, tile_map, n_tiles, I, d, h_bytes, hs_bytes, b.cnt, b.tot, b.off, b.items,
                       static_cast<float*>(y), nullptr, nullptr, nullptr, nullptr);
  else
    hipLaunchKernelGGL((k_ffn_persistent<true, false, uint16_t>), dim3(nb), dim3(P_THREADS), 0, st, h, w2, h_scale,
                       w2_scale, row_token, tile_map, n_tiles, I, d, h_bytes, hs_bytes, b.cnt, b.tot, b.off, b.items,
                       static_cast<uint16_t*>(y), nullptr, nullptr, nullptr, nullptr);
}

}  // namespace moe
