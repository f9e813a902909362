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
// global -> LDS by the direct 16-byte buffer-to-LDS load (two stages; the
// bf16 dgrad keeps three weight stages, dgrad_run_deep; the bf16 wgrad four
// stages of 32 K-rows, wgrad_run).  LDS
// tiles are XOR-swizzled at 16-byte granularity so that fragment reads hit
// distinct banks: K-contiguous tiles as in the forward, M/N-contiguous tiles
// by a XOR of the chunk index that depends on K-row % 4 (mnc_sw).
#include "common.h"

namespace moe {

moe_status quantize_tiles(const void* x, moe_dtype x_t, long long rows, long long cols, int tile_rows, int tile_cols,
                          uint8_t* q, float* scale, void* stream);
long long quantize_runs_max(long long P, int n_seg);
void launch_quantize_runs(const void* x, bool x_f32, long long x_rows, int cols, const int32_t* row_token,
                          bool gather, const int32_t* seg_offset, int n_seg, long long P, int32_t* run_offset,
                          bool offsets, uint8_t* q, float* scale, hipStream_t st, uint8_t* q1, float* s1);

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
  __device__ void issue(uint8_t* st, int wave, int s, uint32_t oob) const { issue_j<0, 8>(st, wave, s, oob); }
  template <int J0, int J1>
  __device__ void issue_j(uint8_t* st, int wave, int s, uint32_t oob) const {
#pragma unroll
    for (int j = J0; j < J1; ++j) dma16(r, st + (wave * 8 + j) * 1024, off[j] | oob, (uint32_t)s * 128u);
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
  __device__ void issue(uint8_t* st, int wave, int s, uint32_t oob) const { issue_j<0, 8>(st, wave, s, oob); }
  template <int J0, int J1>
  __device__ void issue_j(uint8_t* st, int wave, int s, uint32_t oob) const {
#pragma unroll
    for (int j = J0; j < J1; ++j) dma16(r, st + (wave * 8 + j) * 1024, off[j] | oob, (uint32_t)s * kstride);
  }
};

// The K-rows of one segment of the permuted layout (rows seg0 .. seg0 +
// seglen - 1), for both operands of a weight gradient, in stages of WK
// K-rows.  A K-row is live if it lies in the segment and holds a token
// (row_token >= 0); dead K-rows load zeros on both sides.  Operand A reads
// permuted row seg0 + k; operand B the same row, or (GATHER) the token's row
// of x.  Wave w issues the 1 KB blocks g = WNB w .. WNB w + WNB - 1 of each
// operand (block g: K-rows 2 g and 2 g + 1, one per half-wave).  The tokens
// of a stage are loaded into one of four register slots, slot Q for the
// stages k with k % 4 == Q, well before the stage's loads are issued.
constexpr int WK = 32;         // K-rows per wgrad stage
constexpr int WNB = 4;         // 1 KB blocks of each operand per wave and stage
constexpr int WOP = WK * 512;  // bytes of one operand of a stage (16 KB)
constexpr int WST = 2 * WOP;   // bytes of a stage: A, then B
constexpr int WG_VM = 3 * WNB; // global accesses of a wave per stage: tokens + loads of both operands

template <bool GATHER>
struct SegRing {
  __amdgpu_buffer_rsrc_t ra, rb, rt;  // A, B, row_token
  int seglen;
  uint32_t a_rs, b_rs;  // bytes of WK rows of A and of B (the scalar step per stage)
  int kr0;              // K-row of this lane in block j = 0 (block j: kr0 + 2 j)
  uint32_t a_off[WNB];  // byte offset of the lane's chunk of A in stage 0 (row seg0 + kr)
  uint32_t b_off[WNB];  // the same for B (GATHER: column part only; the row comes from the token)
  uint32_t t_off;       // byte offset of the lane's token of block 0 in stage 0
  int tok[4][WNB];
  __device__ void init(int seg0, int seg_len, uint32_t a_rb, uint32_t b_rb, uint32_t a_c, int w, int lane) {
    seglen = seg_len;
    a_rs = a_rb * WK;
    b_rs = b_rb * WK;
    kr0 = 2 * w * WNB + (lane >> 5);
    t_off = (uint32_t)(seg0 + kr0) * 4u;
#pragma unroll
    for (int j = 0; j < WNB; ++j) {
      const int kr = kr0 + 2 * j;
      const uint32_t c16 = (uint32_t)((lane & 31) ^ mnc_sw(kr & 3)) * 16u;
      a_off[j] = (uint32_t)(seg0 + kr) * a_rb + a_c + c16;
      b_off[j] = GATHER ? c16 : (uint32_t)(seg0 + kr) * b_rb + c16;
    }
  }
  // tokens of stage k into slot Q (K-rows past the segment read 0; issue()
  // masks them, so nothing waits for these loads before the stage's issue)
  template <int Q>
  __device__ void fetch(int k) {
    const int lim = seglen - k * WK;  // K-rows of stage k in the segment: kr < lim
#pragma unroll
    for (int j = 0; j < WNB; ++j)
      tok[Q][j] = __builtin_amdgcn_raw_buffer_load_b32(rt, kr0 + 2 * j < lim ? t_off + 8u * j : OOB,
                                                       (uint32_t)(k * WK * 4), 0);
  }
  // stage k of the tile whose B columns start at byte b_c, into stage buffer
  // st (A at st, B at st + WOP); zeros unless live
  template <int Q>
  __device__ void issue(uint8_t* st, int w, int k, uint32_t b_c, bool live) const {
    const int lim = live ? seglen - k * WK : 0;
#pragma unroll
    for (int j = 0; j < WNB; ++j) {
      const int g = w * WNB + j;
      const bool ok = kr0 + 2 * j < lim && tok[Q][j] >= 0;
      const uint32_t oa = ok ? a_off[j] : OOB;
      const uint32_t ob = ok ? (GATHER ? __umul24((uint32_t)tok[Q][j], b_rs / WK) + b_c + b_off[j] : b_off[j] + b_c) : OOB;
      dma16(ra, st + g * 1024, oa, (uint32_t)k * a_rs);
      dma16(rb, st + WOP + g * 1024, ob, GATHER ? 0u : (uint32_t)k * b_rs);
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
// two halves of 128 rows: half h holds the 32-row groups 2 h and 2 h + 1 of
// every wave (buffer row 64 wm + 32 (i - 2 h) + r is tile row
// 128 wm + 32 i + r), so all four waves convert in both halves; 16-byte
// chunk c of buffer row r sits at chunk c ^ (r % 32), so the 32 rows one
// write instruction touches fall on different banks; then every thread
// copies 16-byte chunks out, two full 512-byte rows per wave instruction
// (non-temporal stores).
// Rows >= rows_valid and columns >= cols_valid are not written.
__device__ __forceinline__ void store_tile_bf16(const f32x16_t (&acc)[4][4], uint8_t* __restrict__ stg,
                                                uint16_t* __restrict__ out, long long ld, int rows_valid,
                                                int cols_valid, int wm, int wn, int tid, int lane) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * half + ii;
      const int row = wm * 64 + ii * 32 + (lane & 31);
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
    __syncthreads();
#pragma unroll 4
    for (int rr = 0; rr < 16; ++rr) {
      const int idx = rr * BTHREADS + tid, row = idx >> 5, chunk = idx & 31;
      const uint4 v = *reinterpret_cast<const uint4*>(stg + row * 512 + ((chunk ^ (row & 31)) << 4));
      const int grow = (row >> 6) * 128 + half * 64 + (row & 63);
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


// bf16 dgrad K loop with three weight stages (the forward's layout): LDS
// holds two 32 KB stages of the activation-gradient rows (A) and three of
// the weight K-rows (B), 160 KB; B is loaded two stages ahead and A one, so
// 64 KB of the weight stream is in flight per CU.  The wait before a
// stage's barrier leaves the 8 loads of the B stage two ahead outstanding
// (a wave's loads complete in issue order).  Per stage s:
//   k-step 0: B(s + 2) blocks 0-3 -> b_dst, fragments of k 1, MFMAs of k 0
//   k-step 1: B(s + 2) blocks 4-7, fragments of k 2, MFMAs of k 1
//   k-step 2: fragments of k 3, MFMAs of k 2
//   wait for this wave's LDS reads and everything but B(s + 2), barrier
//   k-step 3: A(s + 2) -> a_cur (the A(s) buffer), fragments of k 0 of
//   stage s + 1 (a_nxt, b_nxt), MFMAs of k 3
// Within a k-step the MFMAs, the LDS reads and the global loads are
// interleaved one by one, so the LDS serves the reads and the
// direct-to-LDS writes while the matrix pipe is busy.
template <int NMFMA, int NDS, int NVM>
__device__ __forceinline__ void dg_order_kstep() {
  constexpr int N = NMFMA > NDS ? (NMFMA > NVM ? NMFMA : NVM) : (NDS > NVM ? NDS : NVM);
#pragma unroll
  for (int q = 0; q < N; ++q) {
    if (q < NMFMA) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (q < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (q < NVM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

// vmcnt(8) / vmcnt(16) and lgkmcnt(0) (expcnt left at its maximum).
constexpr unsigned DG_WAIT_VM8_LGKM0 = (8u & 0xFu) | (0x7u << 4) | ((8u >> 4) << 14);
constexpr unsigned DG_WAIT_VM16_LGKM0 = (16u & 0xFu) | (0x7u << 4) | ((16u >> 4) << 14);

template <int MT>
__device__ __forceinline__ void dg_deep_body(f32x16_t (&acc)[4][4], bf16x8_t (&af)[2][4], bf16x8_t (&bf)[2][4],
                                             const KcRows& A, const MncRows& B, const MncLane& mlb, int wm, int wn,
                                             int lane, int w_wave, int s, uint8_t* __restrict__ a_cur,
                                             const uint8_t* __restrict__ b_cur, const uint8_t* __restrict__ a_nxt,
                                             const uint8_t* __restrict__ b_nxt, uint8_t* __restrict__ b_dst,
                                             uint32_t oob2) {
  constexpr int NM = 4 * MT, ND = MT + 8;
  B.issue_j<0, 4>(b_dst, w_wave, s + 2, oob2);
  load_frags<true, false, 1, MT>(af[1], bf[1], a_cur, b_cur, mlb, mlb, wm, wn, lane);
  mma16<0, MT>(acc, af[0], bf[0]);
  dg_order_kstep<NM, ND, 4>();
  __builtin_amdgcn_sched_barrier(0);
  B.issue_j<4, 8>(b_dst, w_wave, s + 2, oob2);
  load_frags<true, false, 2, MT>(af[0], bf[0], a_cur, b_cur, mlb, mlb, wm, wn, lane);
  mma16<1, MT>(acc, af[1], bf[1]);
  dg_order_kstep<NM, ND, 4>();
  __builtin_amdgcn_sched_barrier(0);
  load_frags<true, false, 3, MT>(af[1], bf[1], a_cur, b_cur, mlb, mlb, wm, wn, lane);
  mma16<2, MT>(acc, af[0], bf[0]);
  dg_order_kstep<NM, ND, 0>();
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(DG_WAIT_VM8_LGKM0);  // own LDS reads done; A(s + 1), B(s + 1) landed
  __builtin_amdgcn_s_barrier();                  // ... for every wave
  __builtin_amdgcn_sched_barrier(0);
  A.issue(a_cur, w_wave, s + 2, oob2);
  load_frags<true, false, 0, MT>(af[0], bf[0], a_nxt, b_nxt, mlb, mlb, wm, wn, lane);
  mma16<3, MT>(acc, af[1], bf[1]);
  dg_order_kstep<NM, ND, 8>();
  __builtin_amdgcn_sched_barrier(0);
}

// K loop and epilogue of one bf16 dgrad item for a wave with MT live 32-row
// groups (all instantiations run the same barriers); lds: DG_LDS bytes, the
// epilogue's staging in its first 64 KB.
constexpr int DG_AB = BT * 128;    // 32 KB: one stage of A or of B
constexpr int DG_LDS = 5 * DG_AB;  // A0 A1 B0 B1 B2
template <bool SWIGLU, typename OT, int MT>
__device__ __forceinline__ void dgrad_run_deep(const KcRows& A, const MncRows& B, uint8_t* __restrict__ lds,
                                               const MncLane& mlb, int wm, int wn, int tid, int lane, int w_wave,
                                               int Kd, int Nd, int n, int row0, int rows,
                                               const uint16_t* __restrict__ ab, OT* __restrict__ out) {
  f32x16_t acc[4][4];
  zero_acc(acc);
  const int nk = Kd / BKS;
  uint8_t* a0 = lds;
  uint8_t* a1 = lds + DG_AB;
  uint8_t* b0 = lds + 2 * DG_AB;
  uint8_t* b1 = lds + 3 * DG_AB;
  uint8_t* b2 = lds + 4 * DG_AB;
  // prologue: A(0), B(0), then B(1), A(1); wait for the first two
  const uint32_t oob1 = nk > 1 ? 0u : OOB;
  A.issue(a0, w_wave, 0, 0u);
  B.issue(b0, w_wave, 0, 0u);
  B.issue(b1, w_wave, 1, oob1);
  A.issue(a1, w_wave, 1, oob1);
  __builtin_amdgcn_s_waitcnt(DG_WAIT_VM16_LGKM0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  bf16x8_t af[2][4], bf[2][4];
  load_frags<true, false, 0, MT>(af[0], bf[0], a0, b0, mlb, mlb, wm, wn, lane);
  for (int s = 0; s < nk; ++s) {
    dg_deep_body<MT>(acc, af, bf, A, B, mlb, wm, wn, lane, w_wave, s, a0, b0, a1, b1, b2, s + 2 < nk ? 0u : OOB);
    uint8_t* t = a0; a0 = a1; a1 = t;
    t = b0; b0 = b1; b1 = b2; b2 = t;
  }
  vm_wait<0>();  // the last (zero) loads land before LDS is reused
  dgrad_epilogue<SWIGLU, OT>(acc, lds, wm, wn, tid, lane, Nd, n, row0, rows, ab, out);
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

// Item order of the dgrad kernels.  The items (row tile, N tile) of one
// expert fill the same range of the item list in any order, since its row
// tiles are contiguous in the tile map.  Inside that range they run in
// groups of up to `grp` row tiles, N-tile major within a group.  The blocks
// of one XCD that run at the same time (about 32, one per CU) then hold up
// to `grp` row tiles of a few N tiles, so each weight slab is read by several
// row tiles together and meets them in L2.  grp = 1 is the tile-major order
// (all N tiles of one row tile, then the next), which already holds 32 / ntn
// row tiles at once; with many N tiles (N = d) it holds about one, and each
// row tile streams the expert's weights from memory again.  dgrad_group
// picks grp from the N-tile count (measured at d = 7168, I = 2048: groups of
// 8 cut the gate/up dgrad by 6-8 %, while at 8 N tiles the tile-major order
// was as fast or faster).
__host__ __device__ constexpr int dgrad_group(int ntn) { return ntn >= 16 ? 8 : 1; }
static_assert(BT == MOE_TILE_ROWS, "a dgrad item covers one tile-map entry");

__device__ __forceinline__ void dgrad_item(long long item, int ntn, int grp, const int32_t* __restrict__ tile_map,
                                           const int32_t* __restrict__ seg_offset, int& tile, int& n) {
  const int tg = (int)(item / ntn);  // some row tile of the same expert
  const int e = tile_map[4LL * tg];
  const int s0 = seg_offset[e];
  const int t0 = tg - ((tile_map[4LL * tg + 1] - s0) / BT);  // the expert's first tile
  const int nt = (seg_offset[e + 1] - s0 + BT - 1) / BT;
  const long long local = item - (long long)t0 * ntn;
  const int g0 = (int)(local / ((long long)grp * ntn)) * grp;
  const int gt = nt - g0 < grp ? nt - g0 : grp;
  const int r = (int)(local - (long long)g0 * ntn);
  n = r / gt;
  tile = t0 + g0 + r % gt;
}

// K loop and epilogue of one E4M3 dgrad item (see dgrad_run_deep).  A stage
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
                                                     const int32_t* __restrict__ n_tiles,
                                                     const int32_t* __restrict__ seg_offset, int Kd, int Nd,
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
  int tile, n;
  dgrad_item(item, ntn, dgrad_group(ntn), tile_map, seg_offset, tile, n);
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
// item list in dgrad_item's order, so the row tiles of one expert, and the
// weight slabs they share, stay in one L2.
//
// SWIGLU: A = dy [P, d] (K = d), W = W2 [E, d, I] (K-rows d, N = I); the
//         epilogue turns dh into [da | db] with the saved [a | b] of the
//         forward and writes dab [P, 2I] (bf16).
// else:   A = dab [P, 2I] (K = 2I), W = W13 [E, 2I, d] (N = d); out = dx [P, d].
template <bool SWIGLU, typename OT>
__global__ __launch_bounds__(BTHREADS) void k_dgrad(const uint16_t* __restrict__ a, const uint16_t* __restrict__ w,
                                                    const int32_t* __restrict__ tile_map,
                                                    const int32_t* __restrict__ n_tiles,
                                                    const int32_t* __restrict__ seg_offset, int Kd, int Nd,
                                                    uint32_t a_bytes, const uint16_t* __restrict__ ab,
                                                    OT* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[DG_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (Nd + BT - 1) / BT;
  const long long items = (long long)(*n_tiles) * ntn;
  const long long q = (items + 7) / 8;
  const long long slot = blockIdx.x >> 3;
  if (slot >= q) return;
  const long long item = (blockIdx.x & 7) * q + slot;
  if (item >= items) return;
  int tile, n;
  dgrad_item(item, ntn, dgrad_group(ntn), tile_map, seg_offset, tile, n);
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
    case 4: dgrad_run_deep<SWIGLU, OT, 4>(A, B, lds, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
    case 3: dgrad_run_deep<SWIGLU, OT, 3>(A, B, lds, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
    case 2: dgrad_run_deep<SWIGLU, OT, 2>(A, B, lds, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
    case 1: dgrad_run_deep<SWIGLU, OT, 1>(A, B, lds, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
    default: dgrad_run_deep<SWIGLU, OT, 0>(A, B, lds, mlb, wm, wn, tid, lane, w_wave, Kd, Nd, n, row0, rows, ab, out); break;
  }
}

// ------------------------------------------------------------- wgrad --
constexpr int WG_STORES = 32;  // buffer stores per wave for one bf16 result tile

// s_waitcnt for at most N global accesses of this wave in flight and none
// of its LDS accesses (expcnt left at its maximum).
template <int N>
__device__ __forceinline__ void vm_lgkm0_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// The fragments of k-step KK of a wgrad stage (both operands M/N-contiguous).
// The stage pointer is a restrict parameter so that these reads carry an
// alias scope of their own, which the direct-to-LDS loads (plain pointers)
// do not share: the compiler then adds no wait of its own on those loads
// before the reads (the explicit waits of wg_stage order them).
template <int KK>
__device__ __forceinline__ void wg_frags(bf16x8_t (&af)[4], bf16x8_t (&bf)[4], const uint8_t* __restrict__ stg,
                                         const MncLane& mla, const MncLane& mlb) {
  af[0] = frag_mnc<0, KK>(stg, mla);
  af[1] = frag_mnc<1, KK>(stg, mla);
  af[2] = frag_mnc<2, KK>(stg, mla);
  af[3] = frag_mnc<3, KK>(stg, mla);
  bf[0] = frag_mnc<0, KK>(stg + WOP, mlb);
  bf[1] = frag_mnc<1, KK>(stg + WOP, mlb);
  bf[2] = frag_mnc<2, KK>(stg + WOP, mlb);
  bf[3] = frag_mnc<3, KK>(stg + WOP, mlb);
}

// One stage k of the wgrad K loop (J = k % 4: stage buffer J, token slot J).
// On entry the fragments of k-step 0 of stage k are in fa[0] / fb[0] and the
// loads of stages k + 1 .. k + 3 are in flight.  The k-step-1 fragments are
// read under the k-step-0 MFMAs; then the wave waits until stage k + 1 has
// landed and its own reads of stage k are done (VMW: the global accesses it
// issued after stage k + 1's loads, which may stay in flight), and the
// barrier makes both hold for every wave.  Buffer J is then free: it takes
// stage k_ld of the tile at column offset b_c (zeros unless live), behind
// the tokens of stage k_tk into slot J + 3; the k-step-0 fragments of stage
// k + 1 are read under the k-step-1 MFMAs.  A stage's loads thus have three
// stages of MFMAs to land, and its tokens (issued three stages before the
// loads that the wait before their use covers) never hold a wait back.
template <bool GATHER, int J, int VMW>
__device__ __forceinline__ void wg_stage(f32x16_t (&acc)[4][4], bf16x8_t (&fa)[2][4], bf16x8_t (&fb)[2][4],
                                         SegRing<GATHER>& S, uint8_t* cur, const uint8_t* nxt, const MncLane& mla,
                                         const MncLane& mlb, int lane, int w_wave, int k_ld, uint32_t b_c, bool live,
                                         int k_tk, bool real) {
  if (real) {
    wg_frags<1>(fa[1], fb[1], cur, mla, mlb);
    mma16<0, 4>(acc, fa[0], fb[0]);
    dg_order_kstep<16, 16, 0>();
  }
  __builtin_amdgcn_sched_barrier(0);
  vm_lgkm0_wait<VMW>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  S.template fetch<(J + 3) & 3>(k_tk);
  S.template issue<J>(cur, w_wave, k_ld, b_c, live);
  if (real) {
    wg_frags<0>(fa[0], fb[0], nxt, mla, mlb);
    mma16<1, 4>(acc, fa[1], fb[1]);
    dg_order_kstep<16, 16, 0>();
  } else {  // a stage of zero K-rows: nothing to multiply
    wg_frags<0>(fa[0], fb[0], nxt, mla, mlb);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Stages kb .. kb + 3 of a tile with nk stages (nk % 4 == 0).  The loads
// issued go to stages kb + 4 .. kb + 7 of this tile, or past its end to
// stages 0 .. 3 of the next tile of the run (bn; zeros after the last);
// tokens are fetched for stages kb + 7 .. kb + 10, taken modulo nk (every
// tile of a run has the same K-rows).  FIRST: the first four stages of a
// tile, whose first three waits may leave the previous tile's WG_STORES
// result stores in flight (issued after the loads they wait for).
template <bool GATHER, bool FIRST>
__device__ __forceinline__ void wg_body(f32x16_t (&acc)[4][4], bf16x8_t (&fa)[2][4], bf16x8_t (&fb)[2][4],
                                        SegRing<GATHER>& S, uint8_t* s0, uint8_t* s1, uint8_t* s2, uint8_t* s3,
                                        const MncLane& mla,
                                        const MncLane& mlb, int lane, int w_wave, int kb, int nk, uint32_t bc,
                                        uint32_t bn, bool more) {
  constexpr int W0 = 2 * WG_VM + (FIRST ? WG_STORES : 0);
  constexpr int W3 = 2 * WG_VM;
  const bool wrap = kb + 4 == nk;
  const int k0 = wrap ? 0 : kb + 4;
  const uint32_t b_c = wrap ? bn : bc;
  const bool live = !wrap || more;
  int kt[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int t = kb + 7 + j;
    t -= t >= nk ? nk : 0;
    t -= t >= nk ? nk : 0;
    kt[j] = t;
  }
  const int nreal = (S.seglen + WK - 1) / WK;  // stages that hold K-rows
  wg_stage<GATHER, 0, W0>(acc, fa, fb, S, s0, s1, mla, mlb, lane, w_wave, k0, b_c, live, kt[0], kb < nreal);
  wg_stage<GATHER, 1, W0>(acc, fa, fb, S, s1, s2, mla, mlb, lane, w_wave, k0 + 1, b_c, live, kt[1], kb + 1 < nreal);
  wg_stage<GATHER, 2, W0>(acc, fa, fb, S, s2, s3, mla, mlb, lane, w_wave, k0 + 2, b_c, live, kt[2], kb + 2 < nreal);
  wg_stage<GATHER, 3, W3>(acc, fa, fb, S, s3, s0, mla, mlb, lane, w_wave, k0 + 3, b_c, live, kt[3], kb + 3 < nreal);
}

// One 256 x 256 result tile of a weight gradient (see mma16 for the
// accumulator layout).  bf16: through stq (32 KB) in four quarters of 64
// rows; quarter qq holds the 32-row group i = qq of every wave: stq row
// 32 wm + r is tile row 128 wm + 32 qq + r, so all four waves convert and
// write their share in every quarter (the conversion is the quarter's
// critical path).  16-byte chunk c of stq row r sits at chunk c ^ (r % 32),
// and every thread then copies 8 chunks out of full 512-byte rows with
// non-temporal buffer stores, exactly WG_STORES per wave (columns past Nd
// are out of range and dropped).  fp32: straight from the accumulators.
template <typename OT>
__device__ __forceinline__ void wgrad_store_tile(f32x16_t (&acc)[4][4], uint8_t* __restrict__ stq, int wm, int wn,
                                                 int tid, int lane, int m, int n, int Md, int Nd,
                                                 OT* __restrict__ ob) {
  if constexpr (sizeof(OT) == 2) {
    // Everything but the loads of the last stage issued (2 WNB) lands
    // before the stores: the tokens the next tile's first stages use are
    // then known to be in registers, and the compiler adds no wait of its
    // own for them behind these stores.
    vm_wait<2 * WNB>();
    const __amdgpu_buffer_rsrc_t ro = rsrc(ob, (uint32_t)Md * (uint32_t)Nd * 2u);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      lds_barrier();
      {
        const int row = wm * 32 + (lane & 31);
        uint8_t* rp = stq + row * 512 + 8 * (lane >> 5);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int chunk = wn * 16 + j * 4 + q;
            const float4 v = acc_get4(acc[qq][j], q);
            lds_st64(rp + ((chunk ^ (row & 31)) << 4), pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
          }
      }
      lds_barrier();
#pragma unroll
      for (int rr = 0; rr < WG_STORES / 4; ++rr) {
        const int idx = rr * BTHREADS + tid, row = idx >> 5, chunk = idx & 31;
        const uint4 v = *reinterpret_cast<const uint4*>(stq + row * 512 + ((chunk ^ (row & 31)) << 4));
        const int grow = m * BT + (row >> 5) * 128 + qq * 32 + (row & 31), gcol = n * BT + chunk * 8;
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

// The K loops and result tiles of one wgrad item (see k_wgrad): the N
// tiles n0 .. n1 - 1 of M tile m, nk stages each (nk % 4 == 0), as one
// stream of stages through four stage buffers, the loads three stages
// ahead across tile boundaries.  A tile's bf16 result stores are issued
// after the loads of the next tile's first four stages and drain under its
// first three stages; fp32 results are waited for at once.
template <bool GATHER, typename OT>
__device__ __forceinline__ void wgrad_run(SegRing<GATHER>& S, uint8_t* st, uint8_t* __restrict__ stq,
                                          const MncLane& mla, const MncLane& mlb, int wm, int wn, int tid, int lane,
                                          int w_wave, int m, int n0, int n1, int nk, int Md, int Nd,
                                          OT* __restrict__ ob) {
  f32x16_t acc[4][4];
  if (nk == 0) {  // no rows: zero tiles
    zero_acc(acc);
    for (int n = n0; n < n1; ++n) wgrad_store_tile(acc, stq, wm, wn, tid, lane, m, n, Md, Nd, ob);
    vm_wait<0>();
    return;
  }
  // prologue: tokens and loads of stages 0 .. 3 (nk >= 4), tokens of stages
  // 4 .. 6 (mod nk), everything landed before the first stage
  const uint32_t bc0 = (uint32_t)n0 * BT * 2u;
  S.template fetch<0>(0);
  S.template fetch<1>(1);
  S.template fetch<2>(2);
  S.template fetch<3>(3);
  S.template issue<0>(st, w_wave, 0, bc0, true);
  S.template issue<1>(st + WST, w_wave, 1, bc0, true);
  S.template issue<2>(st + 2 * WST, w_wave, 2, bc0, true);
  S.template issue<3>(st + 3 * WST, w_wave, 3, bc0, true);
  S.template fetch<0>(4 < nk ? 4 : 0);
  S.template fetch<1>(5 < nk ? 5 : 1);
  S.template fetch<2>(6 < nk ? 6 : 2);
  // The token loads may be moved freely (row_token is read-only); pin them
  // here, so the first stages do not see them as still in flight.
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int j = 0; j < WNB; ++j) asm volatile("" ::"v"(S.tok[q][j]));
  vm_wait<0>();
  lds_barrier();
  bf16x8_t fa[2][4], fb[2][4];
  wg_frags<0>(fa[0], fb[0], st, mla, mlb);
  for (int n = n0; n < n1; ++n) {
    zero_acc(acc);
    const uint32_t bc = (uint32_t)n * BT * 2u, bn = bc + BT * 2u;
    const bool more = n + 1 < n1;
    wg_body<GATHER, true>(acc, fa, fb, S, st, st + WST, st + 2 * WST, st + 3 * WST, mla, mlb, lane, w_wave, 0, nk,
                          bc, bn, more);
    for (int kb = 4; kb < nk; kb += 4)
      wg_body<GATHER, false>(acc, fa, fb, S, st, st + WST, st + 2 * WST, st + 3 * WST, mla, mlb, lane, w_wave, kb,
                             nk, bc, bn, more);
    wgrad_store_tile(acc, stq, wm, wn, tid, lane, m, n, Md, Nd, ob);
    if constexpr (sizeof(OT) != 2) vm_wait<0>();
  }
  vm_wait<0>();  // the last (zero) loads land before the block's LDS is released
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

// The item of this block in a weight-gradient grid: (expert e, M tile m, N
// tiles n0 .. n1 - 1).  Block b runs on XCD b % 8.  XCD x takes every 8th
// shared item (from x), one N tile each, then all items of its routed
// experts (k_wgrad_deal: shares of like row counts), runs of nch N tiles, so
// the blocks that share an expert's rows run together in one L2.  False: the
// block has no item.
__device__ __forceinline__ bool wgrad_item(int E, int Nr, int ntm, int ntn, int nch, const int* __restrict__ deal,
                                           int& e, int& m, int& n0, int& n1) {
  const int runs = (ntn + nch - 1) / nch;  // runs of a routed expert's M tile
  const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int shared_items = (E - Nr) * ntm * ntn;
  const int my_shared = shared_items > x ? (shared_items - x + 7) / 8 : 0;
  if (slot < my_shared) {
    const int item = x + 8 * slot;
    e = Nr + item / (ntm * ntn);
    const int rem = item % (ntm * ntn);
    m = rem / ntn;
    n0 = rem % ntn;
    n1 = n0 + 1;
    return true;
  }
  const int r = slot - my_shared, i = r / (ntm * runs), S = (Nr + 7) / 8;
  // the grid gives every XCD ceil(shared items / 8) shared slots: an XCD
  // with one shared item fewer has one slot past its list (i == S)
  if (i >= S) return false;
  e = deal[x * S + i];
  if (e < 0) return false;
  const int rem = r % (ntm * runs);
  m = rem / runs;
  n0 = (rem % runs) * nch;
  n1 = min(n0 + nch, ntn);
  return true;
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
  // One LDS array for the four stages and the result staging: with two
  // arrays the compiler tags their accesses with alias scopes and then waits
  // for every direct-to-LDS load in flight before each fragment read.
  __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * WST + BOP];
  uint8_t* st = lds;
  uint8_t* stq = lds + 4 * WST;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int e, m, n0, n1;
  if (!wgrad_item(E, Nr, (Md + BT - 1) / BT, (Nd + BT - 1) / BT, nch, deal, e, m, n0, n1)) return;
  const int w_wave = __builtin_amdgcn_readfirstlane(wave);

  SegRing<GATHER> S;
  S.ra = rsrc(a, a_bytes);
  S.rb = rsrc(b, b_bytes);
  S.rt = rsrc(row_token, (uint32_t)P_rows * 4u);
  const int seg0 = seg_offset[e];
  S.init(seg0, seg_offset[e + 1] - seg0, (uint32_t)Md * 2u, (uint32_t)Nd * 2u, (uint32_t)m * BT * 2u, w_wave, lane);

  MncLane mla, mlb;
  mla.init(wm, lane);
  mlb.init(wn, lane);
  OT* ob = out + (long long)e * Md * Nd;
  // Stages rounded up to a multiple of four (the extra stages load zeros),
  // so the loop body (four stages) has no branch on the stage.  No rows:
  // nk = 0 and zeros are stored.
  const int nk = (S.seglen + 4 * WK - 1) / (4 * WK) * 4;
  wgrad_run(S, st, stq, mla, mlb, wm, wn, tid, lane, w_wave, m, n0, n1, nk, Md, Nd, ob);
}

// Blocks of k_wgrad: 8 XCDs x (a share of the shared items + the items of
// ceil(Nr / 8) routed experts).
unsigned wgrad_grid(int Nr, int Ns, int ntm, int ntn, int nch) {
  const long long per_xcd = ceil_div((long long)Ns * ntm * ntn, 8) + ceil_div(Nr, 8) * (long long)ntm * ceil_div(ntn, nch);
  return (unsigned)(8 * per_xcd);
}

// ------------------------------------------------------------ E4M3 wgrad --
// dW_e [M, N] = sum over the rows k of segment e of A[k, :]^T B[k, :] with
// both operands E4M3 codes in the permuted layout (A [P, M], B [P, N];
// padding rows hold code 0) and fp32 power-of-two scales per column and run
// of 128 rows of the segment: scale row run_offset[e] + r of [runs, M] and
// [runs, N], as fp8_quantize_runs writes them.  A stage is one run: 128
// K-rows x 256 columns of each operand, staged M/N-contiguous as the E4M3
// dgrad's weight tiles (MncRows8 layout) and read on both sides with the
// transposing 8-bit LDS read (frag_mnc8), plus the run's scales of the
// tile's 256 + 256 columns.  A fragment lane holds one column (l % 32 of its
// group) for all 64 K of a k-step, all in one run, so the scale of that
// column goes to the matrix instruction per lane as its E8M0 exponent.
constexpr int SC8 = 2 * BOP;             // offset of the A scales in a stage (B scales follow)
constexpr int ST8 = 2 * BOP + 2 * 1024;  // bytes of a stage

struct RunRows8 {
  __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
  int seglen, run0, kr0;
  uint32_t Md, Nd, a_c;   // row bytes of A and B, first column of the A tile
  uint32_t ao[8], bo[8];  // byte offsets of the lane's K-row of load j at run 0 (B: tile column 0)
  // Scale block layout: the scales of tile columns 128 h + 32 i + r
  // (i = 0..3) sit together at float 4 (32 h + r) + i, so a fragment lane
  // reads its four with one 16-byte read.  Lane l of wave w loads float
  // 64 w + l, i.e. column sc_col.
  uint32_t sc_col;
  // Block g = 8 w + j (1 KB) of each operand's stage buffer holds K-rows
  // 4 g .. 4 g + 3: lane l loads K-row kr0 + 4 j (kr0 = 32 w + l / 16),
  // physical chunk l % 16.
  __device__ void init(int seg0, int wave, int lane) {
    kr0 = 32 * wave + (lane >> 4);
    sc_col = (uint32_t)((wave >> 1) * 128 + (lane & 3) * 32 + (wave & 1) * 16 + (lane >> 2));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kr = kr0 + 4 * j;
      const uint32_t c16 = (uint32_t)((lane & 15) ^ f8_sw(kr & 7)) * 16u;
      ao[j] = (uint32_t)(seg0 + kr) * Md + a_c + c16;
      bo[j] = (uint32_t)(seg0 + kr) * Nd + c16;
    }
  }
  // Stage s (run s of the segment) of the N tile whose first column is b_c
  // into st, then the scales of either tile (wave w fills bytes
  // 256 w .. 256 w + 255 of each scale block, see sc_col).  18 global
  // accesses per wave; K-rows past the segment,
  // and every access of a stage that is not live, get an offset with bit 31
  // set, past the buffer, and load zeros (no branch).
  __device__ void issue(uint8_t* st, int wave, int lane, int s, uint32_t b_c, bool live) const {
    const int lim = live ? seglen - s * 128 : 0;  // K-rows kr < lim are live
    const uint32_t sa = (uint32_t)s * 128u * Md, sb = (uint32_t)s * 128u * Nd + b_c;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t oob = ((uint32_t)(kr0 + 4 * j - lim) & 0x80000000u) ^ 0x80000000u;
      dma16(ra, st + (wave * 8 + j) * 1024, (ao[j] + sa) | oob, 0);
      dma16(rb, st + BOP + (wave * 8 + j) * 1024, (bo[j] + sb) | oob, 0);
    }
    const uint32_t run = (uint32_t)(run0 + s);
    const uint32_t soob = live ? 0u : OOB;
    const uint32_t ca = a_c + sc_col, cb = b_c + sc_col;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(st + SC8 + wave * 256), 4, ((run * Md + ca) * 4u) | soob,
                                             0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(st + SC8 + 1024 + wave * 256), 4,
                                             ((run * Nd + cb) * 4u) | soob, 0, 0, 0);
  }
};
constexpr int RUN8_ACCESSES = 18;  // global accesses of RunRows8::issue per wave

// The two k-steps (64 K-rows each) of one stage.
__device__ __forceinline__ void mma_run8(f32x16_t (&acc)[4][4], const uint8_t* st, const MncLane8& mla,
                                         const MncLane8& mlb, int wm, int wn, int lane) {
  const float4 fa = *reinterpret_cast<const float4*>(st + SC8 + 16 * (wm * 32 + (lane & 31)));
  const float4 fb = *reinterpret_cast<const float4*>(st + SC8 + 1024 + 16 * (wn * 32 + (lane & 31)));
  const int ea[4] = {e8m0_of(fa.x), e8m0_of(fa.y), e8m0_of(fa.z), e8m0_of(fa.w)};
  const int eb[4] = {e8m0_of(fb.x), e8m0_of(fb.y), e8m0_of(fb.z), e8m0_of(fb.w)};
  const uint8_t* ta = st;
  const uint8_t* tb = st + BOP;
  i32x8_t a0[4], b0[4], a1[4], b1[4];
  a0[0] = frag_mnc8<0, 0>(ta, mla);
  a0[1] = frag_mnc8<1, 0>(ta, mla);
  a0[2] = frag_mnc8<2, 0>(ta, mla);
  a0[3] = frag_mnc8<3, 0>(ta, mla);
  b0[0] = frag_mnc8<0, 0>(tb, mlb);
  b0[1] = frag_mnc8<1, 0>(tb, mlb);
  b0[2] = frag_mnc8<2, 0>(tb, mlb);
  b0[3] = frag_mnc8<3, 0>(tb, mlb);
  a1[0] = frag_mnc8<0, 1>(ta, mla);
  a1[1] = frag_mnc8<1, 1>(ta, mla);
  a1[2] = frag_mnc8<2, 1>(ta, mla);
  a1[3] = frag_mnc8<3, 1>(ta, mla);
  b1[0] = frag_mnc8<0, 1>(tb, mlb);
  b1[1] = frag_mnc8<1, 1>(tb, mlb);
  b1[2] = frag_mnc8<2, 1>(tb, mlb);
  b1[3] = frag_mnc8<3, 1>(tb, mlb);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b0[j], a0[i], acc[i][j], 0, 0, 0, eb[j], 0, ea[i]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b1[j], a1[i], acc[i][j], 0, 0, 0, eb[j], 0, ea[i]);
  __builtin_amdgcn_sched_barrier(0);
}

// A result tile of one wave (its 128 x 128, see mma16 for the accumulator
// layout; r0, c0: output row and column of its element 0).  bf16: through
// the wave's own 4 KB of LDS, 32 rows x 64 columns at a time, so every lane
// converts its own values in every round (written with lds_st64, which the
// compiler does not order against the direct-to-LDS loads), read back as
// whole 128-byte row pieces and stored with non-temporal buffer stores, 8
// rows per instruction, 32 in all; no workgroup barrier.  Columns past Nd
// are out of range.  fp32: straight from the accumulators.
template <typename OT>
__device__ __forceinline__ void wgrad8_store(const f32x16_t (&acc)[4][4], uint8_t* stw,
                                             OT* ob, int Md, int Nd, int r0, int c0, int lane) {
  if constexpr (sizeof(OT) == 2) {
    // Everything but the loads of the last stage issued (2 WNB) lands
    // before the stores: the tokens the next tile's first stages use are
    // then known to be in registers, and the compiler adds no wait of its
    // own for them behind these stores.
    vm_wait<2 * WNB>();
    const __amdgpu_buffer_rsrc_t ro = rsrc(ob, (uint32_t)Md * (uint32_t)Nd * 2u);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        // round (i, jh): the wave's 32 rows of group i, columns of the MFMA
        // tiles j = 2 jh, 2 jh + 1 (64 columns, 128 bytes a row), every lane
        // converting its own values; chunk c of row r at chunk c ^ (r % 8)
        {
          const int row = lane & 31;
          uint8_t* rp = stw + row * 128 + 8 * (lane >> 5);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int chunk = jj * 4 + q;
              const float4 v = acc_get4(acc[i][2 * jh + jj], q);
              lds_st64(rp + ((chunk ^ (row & 7)) << 4), pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
            }
        }
        // the rows are read back by other lanes: the wave's LDS writes must
        // have completed (measured: without this wait the reads can see
        // the previous round's data)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 8 * r + (lane >> 3), chunk = lane & 7;
          const uint4 v = *reinterpret_cast<const uint4*>(stw + row * 128 + ((chunk ^ (row & 7)) << 4));
          const int grow = r0 + i * 32 + row, gcol = c0 + jh * 64 + chunk * 8;
          const uint32_t off = gcol < Nd ? ((uint32_t)grow * (uint32_t)Nd + (uint32_t)gcol) * 2u : OOB;
          typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
          const u32x4_t w = {v.x, v.y, v.z, v.w};
          __builtin_amdgcn_raw_buffer_store_b128(w, ro, off, 0, 2);  // 2: non-temporal
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + i * 32 + (lane & 31);
      if (r >= Md) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = c0 + j * 32 + 8 * q + 4 * (lane >> 5);
          if (col < Nd) put4(ob + (long long)r * Nd + col, acc_get4(acc[i][j], q));
        }
    }
  }
}

// The next stage to load: N tile ln, run ls.
struct Run8Next {
  int ln, ls;
};

// One stage of an item's sequence (N tiles n0 .. n1 - 1, nk runs each) in
// st: multiply it, wait for the next stage (in the other buffer) and for
// every wave to be done with st, then load the stage after next into st.
// after_store: the first stage of a tile whose predecessor's WG_STORES bf16
// result stores were issued after the loads this wait is for, so it lets
// them stay in flight (the wave's memory operations complete in issue
// order); otherwise the wait is for everything.
__device__ __forceinline__ void wgrad8_step(f32x16_t (&acc)[4][4], uint8_t* st, const RunRows8& S,
                                            const MncLane8& mla, const MncLane8& mlb, Run8Next& nx, int n1, int nk,
                                            int wm, int wn, int lane, int w_wave, bool after_store = false) {
  mma_run8(acc, st, mla, mlb, wm, wn, lane);
  if (after_store)
    vm_wait<WG_STORES>();
  else
    vm_wait<0>();
  lds_barrier();
  S.issue(st, w_wave, lane, nx.ls, (uint32_t)nx.ln * BT, nx.ln < n1);
  if (++nx.ls == nk) {
    nx.ls = 0;
    ++nx.ln;
  }
}

// The nk stages of one N tile (ODD: nk is odd), the first in bufa, then
// alternating.  Every call site names a fixed buffer (no pointer chosen at
// run time), so the compiler knows which buffer each load in flight writes
// and lets the fragment reads of the other one go ahead.
template <bool ODD>
__device__ __forceinline__ void wgrad8_tile(f32x16_t (&acc)[4][4], uint8_t* bufa, uint8_t* bufb, const RunRows8& S,
                                            const MncLane8& mla, const MncLane8& mlb, Run8Next& nx, int n1, int nk,
                                            int wm, int wn, int lane, int w_wave, bool after_store) {
  zero_acc(acc);
  int s = 0;
  if constexpr (ODD) {
    wgrad8_step(acc, bufa, S, mla, mlb, nx, n1, nk, wm, wn, lane, w_wave, after_store);
    for (s = 1; s < nk; s += 2) {
      wgrad8_step(acc, bufb, S, mla, mlb, nx, n1, nk, wm, wn, lane, w_wave);
      wgrad8_step(acc, bufa, S, mla, mlb, nx, n1, nk, wm, wn, lane, w_wave);
    }
  } else {
    wgrad8_step(acc, bufa, S, mla, mlb, nx, n1, nk, wm, wn, lane, w_wave, after_store);
    wgrad8_step(acc, bufb, S, mla, mlb, nx, n1, nk, wm, wn, lane, w_wave);
    for (s = 2; s < nk; s += 2) {
      wgrad8_step(acc, bufa, S, mla, mlb, nx, n1, nk, wm, wn, lane, w_wave);
      wgrad8_step(acc, bufb, S, mla, mlb, nx, n1, nk, wm, wn, lane, w_wave);
    }
  }
}

// The item (expert e, M tile m, N tiles n0 .. n1 - 1) of the E4M3 weight
// gradient, grid and item order as k_wgrad's:
//   down:    A = R(dy) [P, d], B = R(h) [P, I]          -> dW2 [E, d, I]
//   gate/up: A = R([da | db]) [P, 2I], B = R(x) [P, d]  -> dW13 [E, 2I, d]
// (R: runs of 128 rows per column, reading B5; x already gathered into the
// permuted rows by the quantiser).
template <typename OT>
__global__ __launch_bounds__(BTHREADS) void k_wgrad8(const uint8_t* __restrict__ a, const float* __restrict__ as,
                                                     const uint8_t* __restrict__ b, const float* __restrict__ bs,
                                                     const int32_t* __restrict__ seg_offset,
                                                     const int32_t* __restrict__ run_offset, int E, int Nr, int Md,
                                                     int Nd, int nch, uint32_t a_bytes, uint32_t b_bytes,
                                                     uint32_t as_bytes, uint32_t bs_bytes,
                                                     const int* __restrict__ deal, OT* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t st0[ST8];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[ST8];
  __shared__ __attribute__((aligned(1024))) uint8_t stq[4 * 4096];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int e, m, n0, n1;
  if (!wgrad_item(E, Nr, Md / BT, (Nd + BT - 1) / BT, nch, deal, e, m, n0, n1)) return;
  const int w_wave = __builtin_amdgcn_readfirstlane(wave);

  RunRows8 S;
  S.ra = rsrc(a, a_bytes);
  S.rb = rsrc(b, b_bytes);
  S.rsa = rsrc(as, as_bytes);
  S.rsb = rsrc(bs, bs_bytes);
  const int seg0 = seg_offset[e];
  S.seglen = seg_offset[e + 1] - seg0;
  S.run0 = run_offset[e];
  S.Md = (uint32_t)Md;
  S.Nd = (uint32_t)Nd;
  S.a_c = (uint32_t)m * BT;
  S.init(seg0, w_wave, lane);

  MncLane8 mla, mlb;
  mla.init(wm, lane);
  mlb.init(wn, lane);
  uint8_t* stw = stq + w_wave * 4096;
  OT* ob = out + (long long)e * Md * Nd;
  const int nk = S.seglen > 0 ? (S.seglen + 127) / 128 : 0;
  f32x16_t acc[4][4];
  if (nk == 0) {  // no rows: zero tiles
    zero_acc(acc);
    for (int n = n0; n < n1; ++n) wgrad8_store(acc, stw, ob, Md, Nd, m * BT + wm * 128, n * BT + wn * 128, lane);
    vm_wait<0>();
    return;
  }
  // the first two stages (the second may be the first of the next tile)
  S.issue(st0, w_wave, lane, 0, (uint32_t)n0 * BT, true);
  Run8Next nx{nk > 1 ? n0 : n0 + 1, nk > 1 ? 1 : 0};
  S.issue(st1, w_wave, lane, nx.ls, (uint32_t)nx.ln * BT, nx.ln < n1);
  if (++nx.ls == nk) {
    nx.ls = 0;
    ++nx.ln;
  }
  vm_wait<RUN8_ACCESSES>();
  lds_barrier();
  const int r0 = m * BT + wm * 128, c0 = wn * 128;
  // bf16 results leave as exactly WG_STORES stores per wave, which the
  // next tile's first wait lets stay in flight; fp32 ones (a number of
  // stores that depends on the columns) are waited for
  constexpr bool PARTIAL = sizeof(OT) == 2;
  if ((nk & 1) == 0) {
    for (int n = n0; n < n1; ++n) {
      wgrad8_tile<false>(acc, st0, st1, S, mla, mlb, nx, n1, nk, wm, wn, lane, w_wave, PARTIAL && n > n0);
      wgrad8_store(acc, stw, ob, Md, Nd, r0, c0 + n * BT, lane);
    }
  } else {
    // an odd tile ends in the buffer it began with: the next one begins in
    // the other, so tiles go in pairs
    int n = n0;
    for (; n + 1 < n1; n += 2) {
      wgrad8_tile<true>(acc, st0, st1, S, mla, mlb, nx, n1, nk, wm, wn, lane, w_wave, PARTIAL && n > n0);
      wgrad8_store(acc, stw, ob, Md, Nd, r0, c0 + n * BT, lane);
      wgrad8_tile<true>(acc, st1, st0, S, mla, mlb, nx, n1, nk, wm, wn, lane, w_wave, PARTIAL);
      wgrad8_store(acc, stw, ob, Md, Nd, r0, c0 + (n + 1) * BT, lane);
    }
    if (n < n1) {
      wgrad8_tile<true>(acc, st0, st1, S, mla, mlb, nx, n1, nk, wm, wn, lane, w_wave, PARTIAL && n > n0);
      wgrad8_store(acc, stw, ob, Md, Nd, r0, c0 + n * BT, lane);
    }
  }
  vm_wait<0>();
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
    hipLaunchKernelGGL((k_dgrad<true, uint16_t>), dim3(grid), dim3(BTHREADS), 0, st, dy, w2, tile_map, n_tiles,
                       seg_offset, d, I, dy_bytes, ab, dab);
  }
  // dgrad, gate/up: N = d
  {
    const long long items = (long long)tiles_max * (d / BT);
    const unsigned grid = (unsigned)(8 * ((items + 7) / 8));
    hipLaunchKernelGGL((k_dgrad<false, uint16_t>), dim3(grid), dim3(BTHREADS), 0, st, dab, w13, tile_map, n_tiles,
                       seg_offset, 2 * I, d, dab_bytes, nullptr, dx);
  }
  launch_wgrads(x, h, dy, dab, seg_offset, row_token, T, P, d, I, Nr, Ns, deal, dw13, dw2, dw_f32, st);
}

// d <= 16384 and I <= 8192: a lane holds the block scales of two K blocks.
bool ffn_bwd_w8_ok(int d, int I) { return ffn_bwd_ok(d, I) && d / 128 <= 128 && 2 * I / 128 <= 128; }

// Token runs of the weight-gradient products, made while the input-gradient
// products' 1x128 tiles are: run codes and scales of dy and of [da | db],
// the run offsets and what the run quantiser reads besides.
struct RunsOut {
  uint8_t* dyr;
  float* dyrs;
  uint8_t* dabr;
  float* dabrs;
  const int32_t* row_token;
  int32_t* run_offset;
  int n_seg;
};

// The two dgrad products in E4M3: dy and then [da | db] are quantised in
// 1x128 tiles (dyq/dys, dabq/dabs scratch), the weights come as E4M3 codes
// with 128x128 block scales; dab gets [da | db] (bf16), dx the input
// gradient.  With `runs` (and tokens), each of dy and [da | db] is read once
// by the run quantiser, which writes its 128-token runs and its 1x128 tiles
// together.
static void launch_dgrads8(const uint8_t* w13, const float* w13s, const uint8_t* w2, const float* w2s,
                           const uint16_t* ab, const uint16_t* dy, const int32_t* seg_offset,
                           const int32_t* tile_map, const int32_t* n_tiles, int tiles_max, int T, long long P, int d, int I, uint16_t* dab, uint8_t* dyq, float* dys,
                           uint8_t* dabq, float* dabs, uint16_t* dx, hipStream_t st, const RunsOut* runs = nullptr) {
  // with no tokens every row is padding: nothing to quantise (and dy may be NULL)
  if (T > 0 && runs)
    launch_quantize_runs(dy, false, P, d, runs->row_token, false, seg_offset, runs->n_seg, P, runs->run_offset, true,
                         runs->dyr, runs->dyrs, st, dyq, dys);
  else if (T > 0)
    quantize_tiles(dy, MOE_BF16, P, d, 1, 128, dyq, dys, st);
  {
    const long long items = (long long)tiles_max * ((I + BT - 1) / BT);
    const unsigned grid = (unsigned)(8 * ((items + 7) / 8));
    hipLaunchKernelGGL((k_dgrad8<true, uint16_t>), dim3(grid), dim3(BTHREADS), 0, st, dyq, dys, w2, w2s, tile_map,
                       n_tiles, seg_offset, d, I, (uint32_t)(P * d), (uint32_t)(P * (d / 128) * 4), ab, dab);
  }
  if (T > 0 && runs)
    launch_quantize_runs(dab, false, P, 2 * I, runs->row_token, false, seg_offset, runs->n_seg, P, runs->run_offset,
                         false, runs->dabr, runs->dabrs, st, dabq, dabs);
  else if (T > 0)
    quantize_tiles(dab, MOE_BF16, P, 2LL * I, 1, 128, dabq, dabs, st);
  {
    const long long items = (long long)tiles_max * (d / BT);
    const unsigned grid = (unsigned)(8 * ((items + 7) / 8));
    hipLaunchKernelGGL((k_dgrad8<false, uint16_t>), dim3(grid), dim3(BTHREADS), 0, st, dabq, dabs, w13, w13s,
                       tile_map, n_tiles, seg_offset, 2 * I, d, (uint32_t)(P * 2 * I),
                       (uint32_t)(P * (2 * I / 128) * 4), nullptr, dx);
  }
}

// As launch_ffn_bwd_bf16 with the two dgrad products in E4M3
// (launch_dgrads8).  The wgrads stay bf16 (dy and [da | db] unquantised).
void launch_ffn_bwd_w8(const uint16_t* x, const uint8_t* w13, const float* w13s, const uint8_t* w2, const float* w2s,
                       const uint16_t* h, const uint16_t* ab, const uint16_t* dy, const int32_t* seg_offset,
                       const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles, int tiles_max,
                       int T, long long P, int d, int I, int Nr, int Ns, uint16_t* dab, uint8_t* dyq, float* dys,
                       uint8_t* dabq, float* dabs, int* deal, uint16_t* dx, void* dw13, void* dw2, bool dw_f32,
                       hipStream_t st) {
  launch_dgrads8(w13, w13s, w2, w2s, ab, dy, seg_offset, tile_map, n_tiles, tiles_max, T, P, d, I, dab, dyq, dys, dabq, dabs, dx,
                 st);
  launch_wgrads(x, h, dy, dab, seg_offset, row_token, T, P, d, I, Nr, Ns, deal, dw13, dw2, dw_f32, st);
}

// As launch_ffn_bwd_w8 with the weight gradients on E4M3 operands too
// (reading B5): dy, h, [da | db] and the gathered x are quantised in runs of
// 128 rows per column (dy and [da | db] together with their 1x128 tiles for
// the dgrads, so each is read once; dyr, dabr, hr, xr, the four run-scale
// arrays [runs, C] and run_offset [Nr + Ns + 1] are scratch), then k_wgrad8
// makes dW2 and dW13.
void launch_ffn_bwd_f8(const uint16_t* x, const uint8_t* w13, const float* w13s, const uint8_t* w2, const float* w2s,
                       const uint16_t* h, const uint16_t* ab, const uint16_t* dy, const int32_t* seg_offset,
                       const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles, int tiles_max,
                       int T, long long P, int d, int I, int Nr, int Ns, uint16_t* dab, uint8_t* dyq, float* dys,
                       uint8_t* dabq, float* dabs, uint8_t* hr, uint8_t* xr, uint8_t* dyr, uint8_t* dabr,
                       float* dyrs, float* hrs, float* dabrs, float* xrs, int32_t* run_offset, int* deal, uint16_t* dx,
                       void* dw13, void* dw2, bool dw_f32, hipStream_t st) {
  const int E = Nr + Ns;
  const RunsOut ro{dyr, dyrs, dabr, dabrs, row_token, run_offset, E};
  launch_dgrads8(w13, w13s, w2, w2s, ab, dy, seg_offset, tile_map, n_tiles, tiles_max, T, P, d, I, dab, dyq, dys, dabq, dabs, dx,
                 st, &ro);
  if (T <= 0) {  // no 1x128 tiles were made: the runs on their own
    launch_quantize_runs(dy, false, P, d, row_token, false, seg_offset, E, P, run_offset, true, dyr, dyrs, st, nullptr,
                         nullptr);
    launch_quantize_runs(dab, false, P, 2 * I, row_token, false, seg_offset, E, P, run_offset, false, dabr, dabrs, st,
                         nullptr, nullptr);
  }
  launch_quantize_runs(h, false, P, I, row_token, false, seg_offset, E, P, run_offset, false, hr, hrs, st, nullptr,
                       nullptr);
  launch_quantize_runs(x, false, T, d, row_token, true, seg_offset, E, P, run_offset, false, xr, xrs, st, nullptr,
                       nullptr);
  hipLaunchKernelGGL(k_wgrad_deal, dim3(1), dim3(1024), 0, st, seg_offset, Nr, deal);
  const long long runs = quantize_runs_max(P, E);
  const int nch = 4;
  {
    const int ntm = d / BT, ntn = (I + BT - 1) / BT;
    const unsigned grid = wgrad_grid(Nr, Ns, ntm, ntn, nch);
    const uint32_t ab_ = (uint32_t)(P * d), bb = (uint32_t)(P * I), asb = (uint32_t)(runs * d * 4),
                   bsb = (uint32_t)(runs * I * 4);
    if (dw_f32)
      hipLaunchKernelGGL((k_wgrad8<float>), dim3(grid), dim3(BTHREADS), 0, st, dyr, dyrs, hr, hrs, seg_offset,
                         run_offset, E, Nr, d, I, nch, ab_, bb, asb, bsb, deal, static_cast<float*>(dw2));
    else
      hipLaunchKernelGGL((k_wgrad8<uint16_t>), dim3(grid), dim3(BTHREADS), 0, st, dyr, dyrs, hr, hrs, seg_offset,
                         run_offset, E, Nr, d, I, nch, ab_, bb, asb, bsb, deal, static_cast<uint16_t*>(dw2));
  }
  {
    const int ntm = 2 * I / BT, ntn = d / BT;
    const unsigned grid = wgrad_grid(Nr, Ns, ntm, ntn, nch);
    const uint32_t ab_ = (uint32_t)(P * 2 * I), bb = (uint32_t)(P * d), asb = (uint32_t)(runs * 2 * I * 4),
                   bsb = (uint32_t)(runs * d * 4);
    if (dw_f32)
      hipLaunchKernelGGL((k_wgrad8<float>), dim3(grid), dim3(BTHREADS), 0, st, dabr, dabrs, xr, xrs, seg_offset,
                         run_offset, E, Nr, 2 * I, d, nch, ab_, bb, asb, bsb, deal, static_cast<float*>(dw13));
    else
      hipLaunchKernelGGL((k_wgrad8<uint16_t>), dim3(grid), dim3(BTHREADS), 0, st, dabr, dabrs, xr, xrs, seg_offset,
                         run_offset, E, Nr, 2 * I, d, nch, ab_, bb, asb, bsb, deal, static_cast<uint16_t*>(dw13));
  }
}

}  // namespace moe
