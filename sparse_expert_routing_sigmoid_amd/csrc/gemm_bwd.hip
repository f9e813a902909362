// Backward of the grouped SwiGLU expert GEMMs on MFMA (gfx950): bf16, and
// the input-gradient products on E4M3 operands (k_dgrad8, further below).
//
// The forward (expert FFNs of the combine equation, "DeepSeek-V3 Technical
// Report" reading guide, Method section 2, in SwiGLU form) computes per row
// [a | b] = x W13^T, h = SiLU(a) * b, y = h W2^T.  Its gradients, by the
// chain rule, given dy (the gradient reaching y, gate already applied):
//   dh = dy W2                              (dgrad, down)   K = d,  N = I
//   da = dh * b * SiLU'(a),  db = dh * SiLU(a)  (fused into the dgrad epilogue)
//   dx = [da | db] W13                      (dgrad, gate/up) K = 2I, N = d
//   dW2_e  = dy_e^T h_e                     (wgrad, down)   M = d,  N = I, K = rows of e
//   dW13_e = [da | db]_e^T x_e              (wgrad, gate/up) M = 2I, N = d, K = rows of e
//
// The forward multiplies row-major operands that are contiguous along K on
// both sides.  Here one (dgrad) or both (wgrad) operands are contiguous along
// M or N instead.  Such an operand is staged in LDS as it lies in memory
// (64 K-rows of 256 values per stage) and read into MFMA fragments with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16): within each group of 16
// lanes, lane j names the 8 bytes (4 values along M/N) at K-row j / 4 and
// column 4 (j % 4), and lane i receives column i of the four K-rows.  Two such
// reads give a lane the 8 consecutive K values of its column that
// v_mfma_f32_32x32x16_bf16 takes, so no operand is ever transposed in memory.
//
// Block tile 256 x 256 x 64 (K per stage), 4 waves in 2 x 2, each wave
// 128 x 128 as 4 x 4 MFMA tiles of 32x32, fp32 accumulators; operands go
// global -> LDS by the direct 16-byte buffer-to-LDS load, two stages.  LDS
// tiles are XOR-swizzled at 16-byte granularity so that fragment reads hit
// distinct banks: K-contiguous tiles as in the forward, M/N-contiguous tiles
// by a XOR of the chunk index that depends on K-row % 4 (mnc_sw).
#include "common.h"

namespace moe {

moe_status quantize_tiles(const void* x, moe_dtype x_t, long long rows, long long cols, int tile_rows, int tile_cols,
                          uint8_t* q, float* scale, void* stream);

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

constexpr int BT = 256;        // tile rows (M) and columns (N)
constexpr int BKS = 64;        // K values per stage
constexpr int BOP = 32768;     // bytes of one operand per stage
constexpr int BTHREADS = 256;
constexpr uint32_t OOB = 0x80000000u;  // an offset past every buffer: the load writes zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Lane l writes LDS bytes [16 l, 16 l + 16) of the 1 KB block at `lds`.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// K-contiguous tile (256 rows x 128 bytes): fragment of rows r0 .. r0 + 31
// (r0 % 32 == 0) for k-step kk (16 K values): lane l gets row r0 + l % 32,
// K values 8 (l / 32) .. + 7 of the step.
__device__ __forceinline__ bf16x8_t frag_kc(const uint8_t* t, int r0, int kk, int lane) {
  const int c = kk * 2 + (lane >> 5);
  const int sw = (lane & 7) ^ ((lane >> 3) & 1);
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(t + (r0 + (lane & 31)) * 128 + ((c ^ sw) << 4)));
}

// M/N-contiguous tile (64 K-rows x 512 bytes), 16-byte chunk c of K-row kr
// stored at chunk c ^ mnc_sw(kr % 4).  The four K-rows that one transposing
// read touches then fall on distinct banks whether the LDS serves 16 lanes
// over 128 bytes or 32 lanes over 256 bytes per cycle.
__host__ __device__ constexpr int mnc_sw(int y) { return 4 * y + 2 * ((y ^ (y >> 1)) & 1); }

// Fragment reads: the same fragment shape as frag_kc (column c0 + l % 32,
// K values 8 (l / 32) .. + 7 of k-step kk) by two transposing reads of four
// K-rows each.  In a group of 16 lanes, lane j names K-row
// kk * 16 + 8 (group / 2) + j / 4 (+ 4 for the second read) and columns
// c0 + 16 (group % 2) + 4 (j % 4) .. + 3, i.e. logical chunk c0 / 8 + x with
// x = 2 (group % 2) + (j % 4) / 2.  With c0 = 128 wm + 32 i the address splits
// into a lane part per i (MncLane) and a constant, so the reads take
// immediate offsets.
struct MncLane {
  int base[4];  // byte address of the lane's first read for i = 0..3 (wm folded in)
  __device__ void init(int wmn, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int kr = 8 * (g >> 1) + (j >> 2);
    const int x = 2 * (g & 1) + ((j & 3) >> 1);
    const int sw = mnc_sw(j >> 2);  // kr % 4 == j / 4
#pragma unroll
    for (int i = 0; i < 4; ++i) base[i] = kr * 512 + wmn * 256 + ((((4 * i + x) ^ sw)) << 4) + (j & 1) * 8;
  }
};

template <int I, int KK>
__device__ __forceinline__ bf16x8_t frag_mnc(const uint8_t* t, const MncLane& ml) {
  const uint8_t* p = t + ml.base[I] + KK * 8192;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * 512));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// ---------------------------------------------------------- operand loads --
// Instruction j (0..7) of wave w fills the 1 KB block g = 8 w + j of an
// operand's 32 KB stage buffer.

// K-contiguous rows: block g holds tile rows 8 g .. 8 g + 7, lane l row
// 8 g + l / 8, physical chunk l % 8, which holds logical chunk
// (l % 8) ^ (row % 8) ^ ((row / 8) % 2); rows past `rows` load zeros.
struct KcRows {
  __amdgpu_buffer_rsrc_t r;
  uint32_t off[8];
  __device__ void init(const void* base, uint32_t bytes, long long row0, int rows, uint32_t row_bytes, int wave,
                       int lane) {
    r = rsrc(base, bytes);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tr = (wave * 8 + j) * 8 + (lane >> 3);
      const uint32_t c16 = (uint32_t)((lane & 7) ^ (lane >> 3) ^ (j & 1)) * 16u;
      off[j] = tr < rows ? (uint32_t)(row0 + tr) * row_bytes + c16 : OOB;
    }
  }
  __device__ void issue(uint8_t* st, int wave, int s, uint32_t oob) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) dma16(r, st + (wave * 8 + j) * 1024, off[j] | oob, (uint32_t)s * 128u);
  }
};

// M/N-contiguous, K-rows consecutive from the start of the matrix (a weight
// matrix [K, N] of one expert): block g holds K-rows 2 g, 2 g + 1, lane l
// K-row 2 g + l / 32, physical chunk l % 32 = logical chunk ^ mnc_sw(K-row % 4).
struct MncRows {
  __amdgpu_buffer_rsrc_t r;
  uint32_t off[8];
  uint32_t kstride;  // bytes per stage (64 K-rows)
  __device__ void init(const void* base, uint32_t bytes, uint32_t row_bytes, int col0, int wave, int lane) {
    r = rsrc(base, bytes);
    kstride = row_bytes * BKS;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kr = 2 * (wave * 8 + j) + (lane >> 5);
      const uint32_t c = (uint32_t)((lane & 31) ^ mnc_sw(kr & 3));
      off[j] = (uint32_t)kr * row_bytes + (uint32_t)col0 * 2u + c * 16u;
    }
  }
  __device__ void issue(uint8_t* st, int wave, int s, uint32_t oob) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) dma16(r, st + (wave * 8 + j) * 1024, off[j] | oob, (uint32_t)s * kstride);
  }
};

// The K-rows of one segment of the permuted layout (rows seg0 .. seg0 +
// seglen - 1), for both operands of a weight gradient.  A K-row is live if it
// lies in the segment and holds a token (row_token >= 0); dead K-rows load
// zeros on both sides.  Operand A reads permuted row seg0 + k; operand B the
// same row, or (GATHER) the token's row of x.  The loading waves (lw = 0 ..
// 32 / NB - 1) issue NB 1 KB blocks of each operand apiece per stage; the
// tokens of the next stage are fetched one stage ahead.
template <bool GATHER, int NB>
struct SegRows {
  __amdgpu_buffer_rsrc_t ra, rb, rt;  // A, B, row_token
  int seg0, seglen;
  uint32_t a_rb, b_rb, a_c;  // row bytes, A tile column byte offset
  int tok[NB];
  __device__ void fetch(int s, int lw, int lane) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int k = s * BKS + 2 * (lw * NB + j) + (lane >> 5);
      // K-rows past the segment load 0 (out of range); issue() masks them,
      // so nothing here waits for the load
      tok[j] = __builtin_amdgcn_raw_buffer_load_b32(rt, k < seglen ? (uint32_t)(seg0 + k) * 4u : OOB, 0, 0);
    }
  }
  __device__ void issue(uint8_t* sa, uint8_t* sb, int lw, int lane, int s, uint32_t b_c, bool live) const {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int g = lw * NB + j;
      const int kr = 2 * g + (lane >> 5);
      const uint32_t c16 = (uint32_t)((lane & 31) ^ mnc_sw(kr & 3)) * 16u;
      const int row = seg0 + s * BKS + kr;
      const bool ok = live && s * BKS + kr < seglen && tok[j] >= 0;
      const uint32_t oa = ok ? (uint32_t)row * a_rb + a_c + c16 : OOB;
      const uint32_t ob = ok ? (uint32_t)(GATHER ? tok[j] : row) * b_rb + b_c + c16 : OOB;
      dma16(ra, sa + g * 1024, oa, 0);
      dma16(rb, sb + g * 1024, ob, 0);
    }
  }
};

// ------------------------------------------------------------ the K loop --
// Fragments of k-step KK for a wave at (wm, wn): A from the A stage, B from
// the B stage, each K-contiguous (KC) or M/N-contiguous (ml* give the lane
// addresses of the latter).
template <bool A_KC, bool B_KC, int KK, int MT>
__device__ __forceinline__ void load_frags(bf16x8_t (&af)[4], bf16x8_t (&bf)[4], const uint8_t* sa,
                                           const uint8_t* sb, const MncLane& mla, const MncLane& mlb, int wm,
                                           int wn, int lane) {
  if constexpr (A_KC) {
#pragma unroll
    for (int i = 0; i < MT; ++i) af[i] = frag_kc(sa, wm * 128 + i * 32, KK, lane);
  } else {
    static_assert(MT == 4, "M/N-contiguous A tiles are always full");
    af[0] = frag_mnc<0, KK>(sa, mla);
    af[1] = frag_mnc<1, KK>(sa, mla);
    af[2] = frag_mnc<2, KK>(sa, mla);
    af[3] = frag_mnc<3, KK>(sa, mla);
  }
  if constexpr (B_KC) {
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = frag_kc(sb, wn * 128 + j * 32, KK, lane);
  } else {
    bf[0] = frag_mnc<0, KK>(sb, mlb);
    bf[1] = frag_mnc<1, KK>(sb, mlb);
    bf[2] = frag_mnc<2, KK>(sb, mlb);
    bf[3] = frag_mnc<3, KK>(sb, mlb);
  }
}

// The operands go in swapped (B fragment as the matrix instruction's first
// operand), so the instruction computes the tile transposed: lane l holds
// output column-major pieces, element e of acc[i][j] at tile row
// i * 32 + l % 32 and tile column j * 32 + 8 (e / 4) + 4 (l / 32) + e % 4.  Elements 4q ..
// 4q + 3 are then four consecutive output columns of one row, stored with a
// single 8-byte (bf16) or 16-byte (fp32) write.
template <int KK, int MT>
__device__ __forceinline__ void mma16(f32x16_t (&acc)[4][4], const bf16x8_t (&af)[4], const bf16x8_t (&bf)[4]) {
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
}

// The four k-steps of one stage, fragments double-buffered.  MT: the 32-row
// groups of the wave's A rows that hold rows (the others are neither read
// nor multiplied; their accumulators stay zero).
template <bool A_KC, bool B_KC, int MT = 4>
__device__ __forceinline__ void mma_stage(f32x16_t (&acc)[4][4], const uint8_t* __restrict__ sa,
                                          const uint8_t* __restrict__ sb, const MncLane& mla, const MncLane& mlb,
                                          int wm, int wn, int lane) {
  bf16x8_t f0[4], g0[4], f1[4], g1[4];
  load_frags<A_KC, B_KC, 0, MT>(f0, g0, sa, sb, mla, mlb, wm, wn, lane);
  load_frags<A_KC, B_KC, 1, MT>(f1, g1, sa, sb, mla, mlb, wm, wn, lane);
  mma16<0, MT>(acc, f0, g0);
  __builtin_amdgcn_sched_barrier(0);
  load_frags<A_KC, B_KC, 2, MT>(f0, g0, sa, sb, mla, mlb, wm, wn, lane);
  mma16<1, MT>(acc, f1, g1);
  __builtin_amdgcn_sched_barrier(0);
  load_frags<A_KC, B_KC, 3, MT>(f1, g1, sa, sb, mla, mlb, wm, wn, lane);
  mma16<2, MT>(acc, f0, g0);
  __builtin_amdgcn_sched_barrier(0);
  mma16<3, MT>(acc, f1, g1);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

// Elements 4q .. 4q + 3 of an accumulator, read one by one from the
// accumulator registers (left to itself the compiler copies whole
// accumulators to VGPRs first and spills).
__device__ __forceinline__ float4 acc_get4(const f32x16_t& a, int q) {
  float v0, v1, v2, v3;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v0) : "a"(a[4 * q]));
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v1) : "a"(a[4 * q + 1]));
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v2) : "a"(a[4 * q + 2]));
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v3) : "a"(a[4 * q + 3]));
  return make_float4(v0, v1, v2, v3);
}

__device__ __forceinline__ void put4(uint16_t* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}
__device__ __forceinline__ void put4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ float4 get4(const uint16_t* p) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xFFFF0000u), __uint_as_float(q.y << 16),
                     __uint_as_float(q.y & 0xFFFF0000u));
}

// da = dh * b * SiLU'(a), db = dh * SiLU(a), SiLU'(a) = sg (1 + a (1 - sg)),
// sg = sigmoid(a) (hardware exp2 and reciprocal, as the forward's SiLU).
__device__ __forceinline__ void swiglu_bwd(float g, float a, float b, float& da, float& db) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * -1.4426950408889634f));
  da = g * b * sg * (1.0f + a * (1.0f - sg));
  db = g * a * sg;
}

// 16-byte store with the non-temporal hint: results are written once and
// not read again by this kernel (7 % faster over the backward GEMM call than
// plain stores, which allocate the lines in L2).
__device__ __forceinline__ void nt_store16(uint16_t* p, uint4 v) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t q = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(q, reinterpret_cast<u32x4_t*>(p));
}

// 8-byte LDS store written as an instruction of its own: the compiler cannot
// tell that no direct-to-LDS load is still writing the address and would
// otherwise wait for every global access in flight, stores included, first.
// Callers make sure no such load targets the buffer.
__device__ __forceinline__ void lds_st64(uint8_t* p, uint32_t lo, uint32_t hi) {
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)p;
  const unsigned long long v = ((unsigned long long)hi << 32) | lo;
  asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(v) : "memory");
}

// Wait until at most N global accesses of this wave are in flight (they
// complete in issue order).  The builtin, unlike an asm statement, tells the
// compiler what has completed, so it adds no stricter wait of its own for
// registers loaded before.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  // s_waitcnt fields: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that waits only for this wave's LDS accesses.
// __syncthreads() also waits for every global load and store the wave has in
// flight, which would hold a wave's next stage behind its result stores.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// A 256 x 256 bf16 result tile leaves through a free 64 KB stage buffer in
// two halves of 128 rows: the waves of the half write their accumulators as
// bf16 (16-byte chunk c of row r at chunk c ^ (r % 32), so the 32 rows one
// write instruction touches fall on different banks), then every thread
// copies 16-byte chunks out, two full 512-byte rows per wave instruction
// (non-temporal stores).
// Rows >= rows_valid and columns >= cols_valid are not written.
__device__ __forceinline__ void store_tile_bf16(const f32x16_t (&acc)[4][4], uint8_t* __restrict__ stg,
                                                uint16_t* __restrict__ out, long long ld, int rows_valid,
                                                int cols_valid, int wm, int wn, int tid, int lane) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = i * 32 + (lane & 31);
        uint8_t* rp = stg + row * 512 + 8 * (lane >> 5);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int chunk = wn * 16 + j * 4 + q;
            const float4 v = acc_get4(acc[i][j], q);
            *reinterpret_cast<uint2*>(rp + ((chunk ^ (row & 31)) << 4)) =
                make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
          }
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int rr = 0; rr < 16; ++rr) {
      const int idx = rr * BTHREADS + tid, row = idx >> 5, chunk = idx & 31;
      const uint4 v = *reinterpret_cast<const uint4*>(stg + row * 512 + ((chunk ^ (row & 31)) << 4));
      const int grow = half * 128 + row;
      if (grow < rows_valid && chunk * 8 < cols_valid)
        nt_store16(out + grow * ld + chunk * 8, v);
    }
  }
}

// ------------------------------------------------------------- dgrad --
// Epilogue of a dgrad item, shared by the bf16 and E4M3 kernels.
template <bool SWIGLU, typename OT>
__device__ __forceinline__ void dgrad_epilogue(const f32x16_t (&acc)[4][4], uint8_t* __restrict__ st1, int wm, int wn,
                                               int tid, int lane, int Nd, int n, int row0, int rows,
                                               const uint16_t* __restrict__ ab, OT* __restrict__ out) {
  // Epilogue (see mma16 for the accumulator layout): column c of the tile is
  // output column n * 256 + c; rows past the tile's token rows and columns
  // past Nd are not written.  dx goes out through LDS (st1 is free: the last
  // loads went to st0); the SwiGLU backward reads [a | b] and writes
  // [da | db] straight from the accumulators.
  if constexpr (!SWIGLU) {
    store_tile_bf16(acc, st1, reinterpret_cast<uint16_t*>(out) + (long long)row0 * Nd + n * BT, Nd, rows,
                    Nd - n * BT, wm, wn, tid, lane);
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wm * 128 + i * 32 + (lane & 31);
    const bool live = r < rows;
    const long long orow = (long long)row0 + r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n * BT + wn * 128 + j * 32 + 8 * q + 4 * (lane >> 5);
        if (!live || col >= Nd) continue;
        const float4 g = acc_get4(acc[i][j], q);
        {
          const float4 av = get4(ab + orow * 2 * Nd + col);
          const float4 bv = get4(ab + orow * 2 * Nd + Nd + col);
          float4 da, db;
          swiglu_bwd(g.x, av.x, bv.x, da.x, db.x);
          swiglu_bwd(g.y, av.y, bv.y, da.y, db.y);
          swiglu_bwd(g.z, av.z, bv.z, da.z, db.z);
          swiglu_bwd(g.w, av.w, bv.w, da.w, db.w);
          put4(out + orow * 2 * Nd + col, da);
          put4(out + orow * 2 * Nd + Nd + col, db);
        }
      }
  }
}


// K loop and epilogue of one dgrad item for a wave with MT live 32-row
// groups (all instantiations run the same barriers).
template <bool SWIGLU, typename OT, int MT>
__device__ __forceinline__ void dgrad_run(const KcRows& A, const MncRows& B, uint8_t* __restrict__ st0,
                                          uint8_t* __restrict__ st1, const MncLane& mlb, int wm, int wn, int tid,
                                          int lane, int w_wave, int Kd, int Nd, int n, int row0, int rows,
                                          const uint16_t* __restrict__ ab, OT* __restrict__ out) {
  f32x16_t acc[4][4];
  zero_acc(acc);
  // Kd % 128 == 0, so the stage count is even and the loop body, two stages
  // that name their buffers, has no branch: a branch lets the compiler sink
  // MFMAs past the next barrier and costs registers.  The final issue loads
  // zeros (out of range) into a buffer nobody reads.
  const int nk = Kd / BKS;
  A.issue(st0, w_wave, 0, 0u);
  B.issue(st0 + BOP, w_wave, 0, 0u);
  for (int s = 0; s < nk; s += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    A.issue(st1, w_wave, s + 1, 0u);
    B.issue(st1 + BOP, w_wave, s + 1, 0u);
    mma_stage<true, false, MT>(acc, st0, st0 + BOP, mlb, mlb, wm, wn, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const uint32_t oob = s + 2 < nk ? 0u : OOB;
    A.issue(st0, w_wave, s + 2, oob);
    B.issue(st0 + BOP, w_wave, s + 2, oob);
    mma_stage<true, false, MT>(acc, st1, st1 + BOP, mlb, mlb, wm, wn, lane);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  dgrad_epilogue<SWIGLU, OT>(acc, st1, wm, wn, tid, lane, Nd, n, row0, rows, ab, out);
}

// ------------------------------------------------------------ E4M3 dgrad --
// The dgrad products with E4M3 operands: the activation gradient in 1x128
// tiles along K (a power-of-two scale per row and 128 K), the weights in
// 128x128 blocks (one power-of-two scale per block), as the forward's FP8
// path.  A stage is one scale block of K: 128 K values, so a K-contiguous
// row is 128 bytes as in the bf16 kernels (KcRows serves unchanged) and an
// M/N-contiguous weight tile is 128 K-rows of 256 bytes.  The
// v_mfma_scale_f32_32x32x64_f8f6f4 takes, per lane, 32 bytes of K and the
// E8M0 exponent of their scale: the weight block's for the first operand,
// the row's for the second, so the scaling is exact and free.

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;

constexpr int BSC = 1024;  // bytes of the 256 row scales (fp32) of an E4M3 stage

__device__ __forceinline__ int e8m0_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xFF); }

// M/N-contiguous E4M3 tiles (128 K-rows x 256 bytes): 16-byte chunk c of
// K-row kr is stored at chunk c ^ f8_sw(kr % 8).  A transposing 8-bit read
// takes 16 bytes from each of 8 K-rows (16 lanes); with f8_sw the 8 pieces
// fall on distinct banks, and the pieces of two neighbouring lane groups
// (columns +16) on the other 8 chunk positions of a 256-byte row, so the
// read is conflict-free whether the LDS serves 16 lanes over 128 bytes or
// 32 lanes over 256 bytes per cycle.
__host__ __device__ constexpr int f8_sw(int y) { return 2 * y + (y >> 2); }

// Weight loads: block g (1 KB) of the stage holds K-rows 4 g .. 4 g + 3;
// lane l writes K-row 4 g + l / 16, physical chunk l % 16.
struct MncRows8 {
  __amdgpu_buffer_rsrc_t r;
  uint32_t off[8];
  uint32_t kstride;  // bytes per stage (128 K-rows)
  __device__ void init(const void* base, uint32_t bytes, uint32_t row_bytes, int col0, int wave, int lane) {
    r = rsrc(base, bytes);
    kstride = row_bytes * 128u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kr = 4 * (wave * 8 + j) + (lane >> 4);
      const uint32_t c = (uint32_t)((lane & 15) ^ f8_sw(kr & 7));
      off[j] = (uint32_t)kr * row_bytes + (uint32_t)col0 + c * 16u;
    }
  }
  __device__ void issue(uint8_t* st, int wave, int s, uint32_t oob) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) dma16(r, st + (wave * 8 + j) * 1024, off[j] | oob, (uint32_t)s * kstride);
  }
};

// Fragment of the weight tile for MFMA tile jt (columns 32 jt .. + 31 of the
// wave's 128) and k-step kk (64 K): lane l gets column l % 32 and K values
// 32 (l / 32) .. + 31 of the step, in K order, by four transposing reads of
// 8 K-rows.  In a 16-lane group g, lane t names K-row 32 (g / 2) + t / 2
// (+ 8 per read) and 8 bytes at column 16 (g % 2) + 8 (t % 2) of the
// fragment's 32; lane t receives column t of the group's 16, one byte per
// K-row.  The column chunk 8 wn + 2 jt + g % 2 has disjoint bit fields, so
// the swizzled chunk splits into a lane part and 2 jt.
struct MncLane8 {
  int base[4];
  __device__ void init(int wn, int lane) {
    const int g = lane >> 4, t = lane & 15;
    const int kr = 32 * (g >> 1) + (t >> 1);
    const int lx = (wn * 8 + (g & 1)) ^ f8_sw(t >> 1);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) base[jt] = kr * 256 + (((2 * jt) ^ lx) << 4) + 8 * (t & 1);
  }
};

template <int JT, int KK>
__device__ __forceinline__ i32x8_t frag_mnc8(const uint8_t* t, const MncLane8& ml) {
  const uint8_t* p = t + ml.base[JT] + KK * 64 * 256;
  const i32x2_t r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
  const i32x2_t r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 8 * 256));
  const i32x2_t r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 16 * 256));
  const i32x2_t r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 24 * 256));
  const i32x8_t v = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
  return v;
}

// K-contiguous E4M3 rows (the KcRows layout): lane l gets row r0 + l % 32,
// K bytes 32 (l / 32) .. + 31 of k-step kk, the same K order as frag_mnc8.
__device__ __forceinline__ i32x8_t frag_kc8(const uint8_t* t, int r0, int kk, int lane) {
  const int c0 = kk * 4 + 2 * (lane >> 5);
  const int sw = (lane & 7) ^ ((lane >> 3) & 1);
  const uint8_t* row = t + (r0 + (lane & 31)) * 128;
  const uint4 lo = *reinterpret_cast<const uint4*>(row + ((c0 ^ sw) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(row + (((c0 + 1) ^ sw) << 4));
  const i32x8_t v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  return v;
}

// Row scales of the activation tiles: the 256 fp32 scales of a stage's K
// block, 4-byte direct-to-LDS loads, wave w rows 64 w .. 64 w + 63; rows
// past the tile's rows load zeros.
struct RowScales {
  __amdgpu_buffer_rsrc_t r;
  uint32_t off;
  __device__ void init(const float* scales, uint32_t bytes, long long row0, int rows, int nkb, int wave, int lane) {
    r = rsrc(scales, bytes);
    const int tr = wave * 64 + lane;
    off = tr < rows ? (uint32_t)((row0 + tr) * nkb) * 4u : OOB;
  }
  __device__ void issue(uint8_t* sc, int wave, int s, uint32_t oob) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(sc + wave * 256), 4, off | oob, (uint32_t)s * 4u, 0, 0);
  }
};

// The two k-steps of one E4M3 stage.  sb: E8M0 exponent of the wave's weight
// block; the row exponents come from the stage's scale block.
template <int MT>
__device__ __forceinline__ void mma_stage8(f32x16_t (&acc)[4][4], const uint8_t* __restrict__ st, int sb,
                                           const MncLane8& mlb, int wm, int lane) {
  const uint8_t* sa_t = st;
  const uint8_t* sb_t = st + BOP;
  const float* scl = reinterpret_cast<const float*>(st + 2 * BOP);
  int sa[4];
#pragma unroll
  for (int i = 0; i < MT; ++i) sa[i] = e8m0_of(scl[wm * 128 + i * 32 + (lane & 31)]);
  i32x8_t a0[4], b0[4], a1[4], b1[4];
#pragma unroll
  for (int i = 0; i < MT; ++i) a0[i] = frag_kc8(sa_t, wm * 128 + i * 32, 0, lane);
  b0[0] = frag_mnc8<0, 0>(sb_t, mlb);
  b0[1] = frag_mnc8<1, 0>(sb_t, mlb);
  b0[2] = frag_mnc8<2, 0>(sb_t, mlb);
  b0[3] = frag_mnc8<3, 0>(sb_t, mlb);
#pragma unroll
  for (int i = 0; i < MT; ++i) a1[i] = frag_kc8(sa_t, wm * 128 + i * 32, 1, lane);
  b1[0] = frag_mnc8<0, 1>(sb_t, mlb);
  b1[1] = frag_mnc8<1, 1>(sb_t, mlb);
  b1[2] = frag_mnc8<2, 1>(sb_t, mlb);
  b1[3] = frag_mnc8<3, 1>(sb_t, mlb);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b0[j], a0[i], acc[i][j], 0, 0, 0, sb, 0, sa[i]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b1[j], a1[i], acc[i][j], 0, 0, 0, sb, 0, sa[i]);
  __builtin_amdgcn_sched_barrier(0);
}

// K loop and epilogue of one E4M3 dgrad item (see dgrad_run).  A stage
// buffer holds the activation rows (32 KB), the weight K-rows (32 KB) and
// the row scales (1 KB).  Lane l holds the scales of the wave's weight
// blocks for K blocks l and l + 64 (bsc0, bsc1).
template <bool SWIGLU, typename OT, int MT>
__device__ __forceinline__ void dgrad8_run(const KcRows& A, const MncRows8& B, const RowScales& R, float bsc0,
                                           float bsc1, uint8_t* __restrict__ st0, uint8_t* __restrict__ st1,
                                           const MncLane8& mlb, int wm, int wn, int tid, int lane, int w_wave, int Kd,
                                           int Nd, int n, int row0, int rows, const uint16_t* __restrict__ ab,
                                           OT* __restrict__ out) {
  f32x16_t acc[4][4];
  zero_acc(acc);
  // Kd % 256 == 0: an even stage count, a loop body without branches.
  const int nk = Kd / 128;
  auto wscale = [&](int s) {
    const float v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_uint(s < 64 ? bsc0 : bsc1),
                                                                         s & 63));
    return e8m0_of(v);
  };
  A.issue(st0, w_wave, 0, 0u);
  B.issue(st0 + BOP, w_wave, 0, 0u);
  R.issue(st0 + 2 * BOP, w_wave, 0, 0u);
  for (int s = 0; s < nk; s += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    A.issue(st1, w_wave, s + 1, 0u);
    B.issue(st1 + BOP, w_wave, s + 1, 0u);
    R.issue(st1 + 2 * BOP, w_wave, s + 1, 0u);
    mma_stage8<MT>(acc, st0, wscale(s), mlb, wm, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const uint32_t oob = s + 2 < nk ? 0u : OOB;
    A.issue(st0, w_wave, s + 2, oob);
    B.issue(st0 + BOP, w_wave, s + 2, oob);
    R.issue(st0 + 2 * BOP, w_wave, s + 2, oob);
    mma_stage8<MT>(acc, st1, wscale(s + 1), mlb, wm, lane);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  dgrad_epilogue<SWIGLU, OT>(acc, st1, wm, wn, tid, lane, Nd, n, row0, rows, ab, out);
}

// E4M3 dgrad items, dealt as k_dgrad's.  a [P, Kd] E4M3 codes with as
// [P, Kd / 128] fp32 row scales; w [E, Kd, Nd] E4M3 with ws
// [E, Kd / 128, Nd / 128] block scales; the epilogue as k_dgrad's.
template <bool SWIGLU, typename OT>
__global__ __launch_bounds__(BTHREADS) void k_dgrad8(const uint8_t* __restrict__ a, const float* __restrict__ as,
                                                     const uint8_t* __restrict__ w, const float* __restrict__ ws,
                                                     const int32_t* __restrict__ tile_map,
                                                     const int32_t* __restrict__ n_tiles, int Kd, int Nd,
                                                     uint32_t a_bytes, uint32_t as_bytes,
                                                     const uint16_t* __restrict__ ab, OT* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * BOP + BSC];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[2 * BOP + BSC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (Nd + BT - 1) / BT;
  const long long items = (long long)(*n_tiles) * ntn;
  const long long q = (items + 7) / 8;
  const long long slot = blockIdx.x >> 3;
  if (slot >= q) return;
  const long long item = (blockIdx.x & 7) * q + slot;
  if (item >= items) return;
  const int tile = (int)(item / ntn), n = (int)(item % ntn);
  const int4 tm = *reinterpret_cast<const int4*>(tile_map + 4LL * tile);
  const int seg = tm.x, row0 = tm.y, rows = tm.w;
  const int w_wave = __builtin_amdgcn_readfirstlane(wave);
  const int nkb = Kd / 128, nnb = Nd / 128;

  KcRows A;
  A.init(a, a_bytes, row0, rows, (uint32_t)Kd, w_wave, lane);
  MncRows8 B;
  const long long w_expert = (long long)Kd * Nd;
  B.init(w + (long long)seg * w_expert, (uint32_t)w_expert, (uint32_t)Nd, n * BT, w_wave, lane);
  RowScales R;
  R.init(as, as_bytes, row0, rows, nkb, w_wave, lane);
  // the wave's weight blocks: K blocks lane and lane + 64, N block 2 n + wn
  // (past Nd: a block that only dead columns use)
  const int nb = 2 * n + wn;
  const float* wsb = ws + (long long)seg * nkb * nnb + (nb < nnb ? nb : 0);
  const float bsc0 = lane < nkb ? wsb[(long long)lane * nnb] : 1.0f;
  const float bsc1 = lane + 64 < nkb ? wsb[(long long)(lane + 64) * nnb] : 1.0f;

  MncLane8 mlb;
  mlb.init(wn, lane);
  int mt = (rows - wm * 128 + 31) >> 5;
  mt = __builtin_amdgcn_readfirstlane(mt < 0 ? 0 : (mt > 4 ? 4 : mt));
  switch (mt) {
    case 4: dgrad8_run<SWIGLU, OT, 4>(A, B, R, bsc0, bsc1, st0, st1, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
    case 3: dgrad8_run<SWIGLU, OT, 3>(A, B, R, bsc0, bsc1, st0, st1, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
    case 2: dgrad8_run<SWIGLU, OT, 2>(A, B, R, bsc0, bsc1, st0, st1, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
    case 1: dgrad8_run<SWIGLU, OT, 1>(A, B, R, bsc0, bsc1, st0, st1, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
    default: dgrad8_run<SWIGLU, OT, 0>(A, B, R, bsc0, bsc1, st0, st1, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
  }
}

// Items (row tile, N tile) of the tile map, dealt to the XCDs in contiguous
// runs (block b runs on XCD b % 8): XCD x takes items [x q, x q + q) of the
// item list ordered tile-major, so the row tiles of one expert, and the
// weight slabs they share, stay in one L2.
//
// SWIGLU: A = dy [P, d] (K = d), W = W2 [E, d, I] (K-rows d, N = I); the
//         epilogue turns dh into [da | db] with the saved [a | b] of the
//         forward and writes dab [P, 2I] (bf16).
// else:   A = dab [P, 2I] (K = 2I), W = W13 [E, 2I, d] (N = d); out = dx [P, d].
template <bool SWIGLU, typename OT>
__global__ __launch_bounds__(BTHREADS) void k_dgrad(const uint16_t* __restrict__ a, const uint16_t* __restrict__ w,
                                                    const int32_t* __restrict__ tile_map,
                                                    const int32_t* __restrict__ n_tiles, int Kd, int Nd,
                                                    uint32_t a_bytes, const uint16_t* __restrict__ ab,
                                                    OT* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * BOP];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[2 * BOP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (Nd + BT - 1) / BT;
  const long long items = (long long)(*n_tiles) * ntn;
  const long long q = (items + 7) / 8;
  const long long slot = blockIdx.x >> 3;
  if (slot >= q) return;
  const long long item = (blockIdx.x & 7) * q + slot;
  if (item >= items) return;
  const int tile = (int)(item / ntn), n = (int)(item % ntn);
  const int4 tm = *reinterpret_cast<const int4*>(tile_map + 4LL * tile);
  const int seg = tm.x, row0 = tm.y, rows = tm.w;
  const int w_wave = __builtin_amdgcn_readfirstlane(wave);

  KcRows A;
  A.init(a, a_bytes, row0, rows, (uint32_t)Kd * 2u, w_wave, lane);
  MncRows B;
  const long long w_expert = (long long)Kd * Nd * 2;
  B.init(w + (long long)seg * Kd * Nd, (uint32_t)w_expert, (uint32_t)Nd * 2u, n * BT, w_wave, lane);

  MncLane mlb;
  mlb.init(wn, lane);
  // 32-row groups of this wave's rows that hold token rows
  int mt = (rows - wm * 128 + 31) >> 5;
  mt = __builtin_amdgcn_readfirstlane(mt < 0 ? 0 : (mt > 4 ? 4 : mt));
  switch (mt) {
    case 4: dgrad_run<SWIGLU, OT, 4>(A, B, st0, st1, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
    case 3: dgrad_run<SWIGLU, OT, 3>(A, B, st0, st1, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
    case 2: dgrad_run<SWIGLU, OT, 2>(A, B, st0, st1, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
    case 1: dgrad_run<SWIGLU, OT, 1>(A, B, st0, st1, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
    default: dgrad_run<SWIGLU, OT, 0>(A, B, st0, st1, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
  }
}

// ------------------------------------------------------------- wgrad --
constexpr int WG_STORES = 32;  // buffer stores per wave for one bf16 result tile

// One pair of stages of a wgrad K loop.  On entry st0 holds stage s
// (complete and visible) and the loads of stage s + 1 into st1 are in
// flight, issued before the last `pending` global accesses of this wave;
// `tok` holds the tokens of stage (s + 2) % nk.  Each buffer is refilled as
// soon as every wave has read it: with the stage after next of this N tile,
// or past its last stage the first stages of the next N tile of the run
// (zeros after the last).
template <int PENDING, bool GATHER>
__device__ __forceinline__ void wgrad_pair(f32x16_t (&acc)[4][4], SegRows<GATHER, 8>& S, uint8_t* __restrict__ st0,
                                           uint8_t* __restrict__ st1, const MncLane& mla, const MncLane& mlb, int wm,
                                           int wn, int lane, int w_wave, int s, int nk, uint32_t bc, bool more) {
  const bool wrap = s + 2 == nk;
  const uint32_t bn = wrap ? bc + BT * 2u : bc;
  const bool live = !wrap || more;
  mma_stage<false, false>(acc, st0, st0 + BOP, mla, mlb, wm, wn, lane);
  vm_wait<PENDING>();
  lds_barrier();
  S.issue(st0, st0 + BOP, w_wave, lane, wrap ? 0 : s + 2, bn, live);
  S.fetch(wrap ? 1 : s + 3, w_wave, lane);
  mma_stage<false, false>(acc, st1, st1 + BOP, mla, mlb, wm, wn, lane);
  vm_wait<0>();
  lds_barrier();
  S.issue(st1, st1 + BOP, w_wave, lane, wrap ? 1 : s + 3, bn, live);
  S.fetch(wrap ? (2 < nk ? 2 : 0) : (s + 4 < nk ? s + 4 : 0), w_wave, lane);
}

// The K loops and result tiles of one wgrad item (see k_wgrad).  bf16 result
// tiles leave through a third LDS buffer (stq, 32 KB) in four quarters of 64
// rows, so both stage buffers keep loading meanwhile: the tile's stores are
// issued after the loads of the next tile's first two stages and only the
// wait for the second of those (vmcnt counts in issue order) lets them
// drain, a whole stage of MFMAs later.
template <bool GATHER, typename OT>
__device__ __forceinline__ void wgrad_run(SegRows<GATHER, 8>& S, uint8_t* __restrict__ st0, uint8_t* __restrict__ st1,
                                          uint8_t* __restrict__ stq, const MncLane& mla, const MncLane& mlb, int wm,
                                          int wn, int tid, int lane, int w_wave, int m, int n0, int n1, int nk, int Md,
                                          int Nd, OT* __restrict__ ob) {
  constexpr bool BF16 = sizeof(OT) == 2;
  S.fetch(0, w_wave, lane);
  S.issue(st0, st0 + BOP, w_wave, lane, 0, (uint32_t)n0 * BT * 2u, nk > 0);
  S.fetch(1, w_wave, lane);
  S.issue(st1, st1 + BOP, w_wave, lane, 1, (uint32_t)n0 * BT * 2u, nk > 0);
  S.fetch(2 < nk ? 2 : 0, w_wave, lane);
  // The token loads may be moved freely (row_token is read-only); pin them
  // here, so the first pair does not see them as still in flight.
#pragma unroll
  for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(S.tok[j]));
  vm_wait<0>();
  lds_barrier();
  for (int n = n0; n < n1; ++n) {
    f32x16_t acc[4][4];
    zero_acc(acc);
    const uint32_t bc = (uint32_t)n * BT * 2u;
    const bool more = n + 1 < n1;
    // The first pair runs with the previous tile's stores still in flight.
    // Its stage index is hidden from the compiler: as a constant it would
    // hoist that pair's load addresses out of the N loop and spill them,
    // and a reload from scratch would wait for the stores.
    int s0 = 0;
    asm volatile("" : "+s"(s0));
    if (nk > 0)
      wgrad_pair<BF16 ? WG_STORES : 0>(acc, S, st0, st1, mla, mlb, wm, wn, lane, w_wave, s0, nk, bc, more);
    for (int s = 2; s < nk; s += 2)
      wgrad_pair<0>(acc, S, st0, st1, mla, mlb, wm, wn, lane, w_wave, s, nk, bc, more);
    // (see mma16 for the accumulator layout)
    if constexpr (BF16) {
      // quarter qq: rows 64 qq .. 64 qq + 63 of the tile, held by the waves
      // with wm = qq / 2 as their 32-row groups i = 2 (qq % 2), + 1; 16-byte
      // chunk c of row r at chunk c ^ (r % 32); every thread then copies 8
      // chunks out of full 512-byte rows with non-temporal buffer stores
      // (columns past Nd are out of range and dropped).
      const __amdgpu_buffer_rsrc_t ro = rsrc(ob, (uint32_t)Md * (uint32_t)Nd * 2u);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        lds_barrier();
        if (wm == qq / 2) {
#pragma unroll
          for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * (qq % 2) + ii;
            const int row = ii * 32 + (lane & 31);
            uint8_t* rp = stq + row * 512 + 8 * (lane >> 5);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int chunk = wn * 16 + j * 4 + q;
                const float4 v = acc_get4(acc[i][j], q);
                lds_st64(rp + ((chunk ^ (row & 31)) << 4), pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
              }
          }
        }
        lds_barrier();
#pragma unroll
        for (int rr = 0; rr < WG_STORES / 4; ++rr) {
          const int idx = rr * BTHREADS + tid, row = idx >> 5, chunk = idx & 31;
          const uint4 v = *reinterpret_cast<const uint4*>(stq + row * 512 + ((chunk ^ (row & 31)) << 4));
          const int grow = m * BT + qq * 64 + row, gcol = n * BT + chunk * 8;
          const uint32_t off = grow < Md && gcol < Nd ? ((uint32_t)grow * (uint32_t)Nd + (uint32_t)gcol) * 2u : OOB;
          typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
          const u32x4_t q = {v.x, v.y, v.z, v.w};
          __builtin_amdgcn_raw_buffer_store_b128(q, ro, off, 0, 2);  // 2: non-temporal
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m * BT + wm * 128 + i * 32 + (lane & 31);
        if (r >= Md) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = n * BT + wn * 128 + j * 32 + 8 * q + 4 * (lane >> 5);
            if (col < Nd) put4(ob + (long long)r * Nd + col, acc_get4(acc[i][j], q));
          }
      }
    }
  }
}

// The routed experts of the wgrad dealt to the 8 XCDs by their (padded)
// row counts: ranked largest first (ties: lower index first), dealt in
// snake rounds (0..7, 7..0, ...), so every XCD gets a like share of the
// rows.  deal[x * S + i] is XCD x's i-th expert, -1 past its last;
// S = ceil(Nr / 8).  One block; Nr <= 1024.
__global__ __launch_bounds__(1024) void k_wgrad_deal(const int32_t* __restrict__ seg_offset, int Nr,
                                                     int* __restrict__ deal) {
  __shared__ int s_len[1024];
  const int S = (Nr + 7) / 8;
  for (int v = threadIdx.x; v < Nr; v += 1024) s_len[v] = seg_offset[v + 1] - seg_offset[v];
  for (int q = threadIdx.x; q < 8 * S; q += 1024) deal[q] = -1;
  __syncthreads();
  for (int v = threadIdx.x; v < Nr; v += 1024) {
    const int lv = s_len[v];
    int rank = 0;
    for (int w = 0; w < Nr; ++w) rank += (s_len[w] > lv) || (s_len[w] == lv && w < v);
    const int i = rank >> 3, k = rank & 7;
    deal[((i & 1) ? 7 - k : k) * S + i] = v;
  }
}

// dW_e [M, N] = A_e^T B_e over the K-rows of segment e.  An item is (expert,
// M tile, run of N tiles): one block computes the N tiles of the run one
// after the other with the same K-rows (the tokens are fetched once per
// stage index, the A tile is re-read from L2); the first stage of the next
// N tile is loaded while the last stage of the current one is multiplied,
// and a tile's results are stored while the next one is multiplied
// (wgrad_run).  Routed experts (a few rows each) take runs of `nch` N tiles;
// shared experts (every token) one N tile per item, and go first.
// DOWN:  A = dy [P, d] (M = d), B = h [P, I] (N = I)   -> dW2 [E, d, I]
// !DOWN: A = dab [P, 2I] (M = 2I), B = x [T, d] gathered by row_token (N = d)
//        -> dW13 [E, 2I, d]
template <bool GATHER, typename OT>
__global__ __launch_bounds__(BTHREADS) void k_wgrad(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                                                    const int32_t* __restrict__ seg_offset,
                                                    const int32_t* __restrict__ row_token, int P_rows, int E, int Nr,
                                                    int Md, int Nd, int nch, uint32_t a_bytes, uint32_t b_bytes,
                                                    const int* __restrict__ deal, OT* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * BOP];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[2 * BOP];
  __shared__ __attribute__((aligned(1024))) uint8_t stq[BOP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntm = (Md + BT - 1) / BT, ntn = (Nd + BT - 1) / BT;
  const int runs = (ntn + nch - 1) / nch;  // runs of a routed expert's M tile
  // Block b runs on XCD b % 8.  XCD x takes every 8th shared item (from x),
  // then all items of its routed experts (k_wgrad_deal: shares of like row
  // counts), so the blocks that share an expert's rows run together in one
  // L2.
  const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int shared_items = (E - Nr) * ntm * ntn;
  const int my_shared = shared_items > x ? (shared_items - x + 7) / 8 : 0;
  int e, m, n0, n1;
  if (slot < my_shared) {
    const int item = x + 8 * slot;
    e = Nr + item / (ntm * ntn);
    const int rem = item % (ntm * ntn);
    m = rem / ntn;
    n0 = rem % ntn;
    n1 = n0 + 1;
  } else {
    const int r = slot - my_shared, i = r / (ntm * runs), S = (Nr + 7) / 8;
    // the grid gives every XCD ceil(shared items / 8) shared slots: an XCD
    // with one shared item fewer has one slot past its list (i == S)
    if (i >= S) return;
    e = deal[x * S + i];
    if (e < 0) return;
    const int rem = r % (ntm * runs);
    m = rem / runs;
    n0 = (rem % runs) * nch;
    n1 = min(n0 + nch, ntn);
  }
  const int w_wave = __builtin_amdgcn_readfirstlane(wave);

  SegRows<GATHER, 8> S;
  S.ra = rsrc(a, a_bytes);
  S.rb = rsrc(b, b_bytes);
  S.rt = rsrc(row_token, (uint32_t)P_rows * 4u);
  S.seg0 = seg_offset[e];
  S.seglen = seg_offset[e + 1] - S.seg0;
  S.a_rb = (uint32_t)Md * 2u;
  S.b_rb = (uint32_t)Nd * 2u;
  S.a_c = (uint32_t)m * BT * 2u;

  MncLane mla, mlb;
  mla.init(wm, lane);
  mlb.init(wn, lane);
  OT* ob = out + (long long)e * Md * Nd;
  // Stages rounded up to an even count (the extra stage loads zeros), so the
  // two-stage loop body has no branch on the stage.  No rows: nk = 0 and
  // zeros are stored.
  const int nk = (S.seglen + 2 * BKS - 1) / (2 * BKS) * 2;
  wgrad_run(S, st0, st1, stq, mla, mlb, wm, wn, tid, lane, w_wave, m, n0, n1, nk, Md, Nd, ob);
}

// Blocks of k_wgrad: 8 XCDs x (a share of the shared items + the items of
// ceil(Nr / 8) routed experts).
unsigned wgrad_grid(int Nr, int Ns, int ntm, int ntn, int nch) {
  const long long per_xcd = ceil_div((long long)Ns * ntm * ntn, 8) + ceil_div(Nr, 8) * (long long)ntm * ceil_div(ntn, nch);
  return (unsigned)(8 * per_xcd);
}

}  // namespace

// d % 256 and I % 128: full M tiles, even stage counts (Kd % 128 == 0).
bool ffn_bwd_ok(int d, int I) { return d % 256 == 0 && I % 128 == 0; }

// Both weight gradients (bf16 operands): dW2 [E, d, I] and dW13 [E, 2I, d]
// in dw_f32 ? fp32 : bf16, routed runs of 4 N tiles.
static void launch_wgrads(const uint16_t* x, const uint16_t* h, const uint16_t* dy, const uint16_t* dab,
                          const int32_t* seg_offset, const int32_t* row_token, int T, long long P, int d, int I,
                          int Nr, int Ns, int* deal, void* dw13, void* dw2, bool dw_f32, hipStream_t st) {
  const int E = Nr + Ns;
  hipLaunchKernelGGL(k_wgrad_deal, dim3(1), dim3(1024), 0, st, seg_offset, Nr, deal);
  const uint32_t dy_bytes = (uint32_t)(P * d * 2), dab_bytes = (uint32_t)(P * 2 * I * 2);
  const uint32_t h_bytes = (uint32_t)(P * I * 2), x_bytes = (uint32_t)((long long)T * d * 2);
  {
    const int ntm = d / BT, ntn = (I + BT - 1) / BT, nch = 4;
    const unsigned grid = wgrad_grid(Nr, Ns, ntm, ntn, nch);
    if (dw_f32)
      hipLaunchKernelGGL((k_wgrad<false, float>), dim3(grid), dim3(BTHREADS), 0, st, dy, h, seg_offset, row_token,
                         (int)P, E, Nr, d, I, nch, dy_bytes, h_bytes, deal, static_cast<float*>(dw2));
    else
      hipLaunchKernelGGL((k_wgrad<false, uint16_t>), dim3(grid), dim3(BTHREADS), 0, st, dy, h, seg_offset, row_token,
                         (int)P, E, Nr, d, I, nch, dy_bytes, h_bytes, deal, static_cast<uint16_t*>(dw2));
  }
  {
    const int ntm = 2 * I / BT, ntn = d / BT, nch = 4;
    const unsigned grid = wgrad_grid(Nr, Ns, ntm, ntn, nch);
    if (dw_f32)
      hipLaunchKernelGGL((k_wgrad<true, float>), dim3(grid), dim3(BTHREADS), 0, st, dab, x, seg_offset, row_token,
                         (int)P, E, Nr, 2 * I, d, nch, dab_bytes, x_bytes, deal, static_cast<float*>(dw13));
    else
      hipLaunchKernelGGL((k_wgrad<true, uint16_t>), dim3(grid), dim3(BTHREADS), 0, st, dab, x, seg_offset, row_token,
                         (int)P, E, Nr, 2 * I, d, nch, dab_bytes, x_bytes, deal, static_cast<uint16_t*>(dw13));
  }
}

// dy [P, d], ab [P, 2I], h [P, I] (bf16, the forward's), x [T, d]; dab is
// scratch [P, 2I]; dx [P, d] bf16; dW13 [E, 2I, d], dW2 [E, d, I] in dw_f32 ?
// fp32 : bf16.
void launch_ffn_bwd_bf16(const uint16_t* x, const uint16_t* w13, const uint16_t* w2, const uint16_t* h,
                         const uint16_t* ab, const uint16_t* dy, const int32_t* seg_offset, const int32_t* row_token,
                         const int32_t* tile_map, const int32_t* n_tiles, int tiles_max, int T, long long P, int d,
                         int I, int Nr, int Ns, uint16_t* dab, int* deal, uint16_t* dx, void* dw13, void* dw2,
                         bool dw_f32, hipStream_t st) {
  const uint32_t dy_bytes = (uint32_t)(P * d * 2), dab_bytes = (uint32_t)(P * 2 * I * 2);
  // dgrad, down + SwiGLU: N = I
  {
    const long long items = (long long)tiles_max * ((I + BT - 1) / BT);
    const unsigned grid = (unsigned)(8 * ((items + 7) / 8));
    hipLaunchKernelGGL((k_dgrad<true, uint16_t>), dim3(grid), dim3(BTHREADS), 0, st, dy, w2, tile_map, n_tiles, d, I,
                       dy_bytes, ab, dab);
  }
  // dgrad, gate/up: N = d
  {
    const long long items = (long long)tiles_max * (d / BT);
    const unsigned grid = (unsigned)(8 * ((items + 7) / 8));
    hipLaunchKernelGGL((k_dgrad<false, uint16_t>), dim3(grid), dim3(BTHREADS), 0, st, dab, w13, tile_map, n_tiles,
                       2 * I, d, dab_bytes, nullptr, dx);
  }
  launch_wgrads(x, h, dy, dab, seg_offset, row_token, T, P, d, I, Nr, Ns, deal, dw13, dw2, dw_f32, st);
}

// d <= 16384 and I <= 8192: a lane holds the block scales of two K blocks.
bool ffn_bwd_w8_ok(int d, int I) { return ffn_bwd_ok(d, I) && d / 128 <= 128 && 2 * I / 128 <= 128; }

// As launch_ffn_bwd_bf16 with the two dgrad products in E4M3: dy and then
// [da | db] are quantised in 1x128 tiles (dyq/dys, dabq/dabs scratch), the
// weights come as E4M3 codes with 128x128 block scales.  The wgrads stay
// bf16 (dy and [da | db] unquantised).
void launch_ffn_bwd_w8(const uint16_t* x, const uint8_t* w13, const float* w13s, const uint8_t* w2, const float* w2s,
                       const uint16_t* h, const uint16_t* ab, const uint16_t* dy, const int32_t* seg_offset,
                       const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles, int tiles_max,
                       int T, long long P, int d, int I, int Nr, int Ns, uint16_t* dab, uint8_t* dyq, float* dys,
                       uint8_t* dabq, float* dabs, int* deal, uint16_t* dx, void* dw13, void* dw2, bool dw_f32,
                       hipStream_t st) {
  // with no tokens every row is padding: nothing to quantise (and dy may be NULL)
  if (T > 0) quantize_tiles(dy, MOE_BF16, P, d, 1, 128, dyq, dys, st);
  {
    const long long items = (long long)tiles_max * ((I + BT - 1) / BT);
    const unsigned grid = (unsigned)(8 * ((items + 7) / 8));
    hipLaunchKernelGGL((k_dgrad8<true, uint16_t>), dim3(grid), dim3(BTHREADS), 0, st, dyq, dys, w2, w2s, tile_map,
                       n_tiles, d, I, (uint32_t)(P * d), (uint32_t)(P * (d / 128) * 4), ab, dab);
  }
  if (T > 0) quantize_tiles(dab, MOE_BF16, P, 2LL * I, 1, 128, dabq, dabs, st);
  {
    const long long items = (long long)tiles_max * (d / BT);
    const unsigned grid = (unsigned)(8 * ((items + 7) / 8));
    hipLaunchKernelGGL((k_dgrad8<false, uint16_t>), dim3(grid), dim3(BTHREADS), 0, st, dabq, dabs, w13, w13s,
                       tile_map, n_tiles, 2 * I, d, (uint32_t)(P * 2 * I), (uint32_t)(P * (2 * I / 128) * 4), nullptr,
                       dx);
  }
  launch_wgrads(x, h, dy, dab, seg_offset, row_token, T, P, d, I, Nr, Ns, deal, dw13, dw2, dw_f32, st);
}

}  // namespace moe
