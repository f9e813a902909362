/*
 * moe_mi355x.h - C ABI of the DeepSeekMoE layer forward on AMD MI355X (gfx950).
 *
 * The layer (sources: the "DeepSeek-V3 Technical Report" reading guide on
 * xyznot.com, Turkish edition "Okuma rehberi" and French edition "Guide de
 * lecture", Method section 2 "DeepSeekMoE with auxiliary-loss-free
 * balancing", cited below as [RG-MoE]; its "Key ideas" section, FP8 bullet,
 * cited as [RG-FP8]):
 *
 *   s_{i,t}  = Sigmoid(u_t . e_i)                       affinity sentence
 *   g'_{i,t} = s_{i,t} if s_{i,t}+b_i is in the Top-K   gate equation
 *              of {s_{j,t}+b_j}, else 0; g = g' normalised
 *   h'_t     = u_t + sum_j FFN^(s)_j(u_t)                combine equation
 *              + sum_i g_{i,t} FFN^(r)_i(u_t)
 *   b_i     <- b_i - gamma if expert i is overloaded,    bias rule
 *              b_i + gamma if underloaded (gamma = 0.001)
 *
 * One forward is: moe_route -> moe_permute -> [fp8_quantize_tiles] ->
 * moe_expert_gemm -> moe_combine, then moe_bias_update at the end of a step.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named as device pointers must point to device memory (HBM) of
 *    the current HIP device; the caller owns every buffer.  The library
 *    allocates and frees no memory, keeps no pointer after a call returns
 *    and holds no state between calls (no stream, event, lock or cache of
 *    its own), except moe_permute_noalloc's device array and its address
 *    per GPU.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call
 *    enqueues its kernels on it and returns without synchronising; calls on
 *    distinct streams may run concurrently from different threads.
 *  - Tensors are row-major and contiguous, element offsets are 64-bit.
 *    Data tensors (u, centroids, x, weights, y, out, q and the workspaces)
 *    must be 16-byte aligned (hipMalloc and torch allocations are 256-byte
 *    aligned); index, gate, load, bias and scale arrays need only the
 *    alignment of their element type.  A misaligned data tensor is
 *    MOE_EINVAL.
 *    bf16 is stored as raw 16-bit patterns, E4M3 as one byte per value (OCP
 *    E4M3FN: exponent bias 7, largest finite 448, no infinities).
 *  - Arguments are checked on the host before any launch.  A bad argument
 *    returns MOE_EINVAL (or MOE_EUNSUPPORTED / MOE_EWORKSPACE) and launches
 *    nothing; a launch failure returns MOE_EHIP.  With valid arguments the
 *    device code cannot fail.  moe_last_error() gives a message for the last
 *    failing call of the calling thread.  Device data (indices, counts) is
 *    not validated: it must come from the producing entry point.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

/* Limits of this implementation. */
#define MOE_MAX_EXPERTS 1024   /* routed + shared experts */
#define MOE_MAX_K 16           /* routed experts per token */
#define MOE_TILE_ROWS 256      /* rows per entry of the GEMM tile map */

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* NULL pointer, size out of range, bad enum */
  MOE_EUNSUPPORTED = 2,  /* a valid combination the library does not run */
  MOE_EWORKSPACE = 3,    /* workspace smaller than the size helper returns */
  MOE_EHIP = 4           /* the HIP runtime reported an error at launch */
} moe_status;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_E4M3 = 2
} moe_dtype;

/* Flags of moe_combine: drop a term of the combine equation (component checks). */
#define MOE_COMBINE_NO_RESIDUAL 1u
#define MOE_COMBINE_NO_SHARED 2u
#define MOE_COMBINE_NO_ROUTED 4u

int moe_abi_version(void);
const char* moe_status_str(int status);
/* Message of the last failing call made by this thread ("" if none). */
const char* moe_last_error(void);

/* ------------------------------------------------------------------------
 * moe_route: sigmoid affinities, bias-steered top-K, normalised gates, loads.
 * [RG-MoE] affinity sentence and gate equation.
 *
 *   u          device [T, d], dtype u_t (MOE_F32 or MOE_BF16): token states
 *   centroids  device [Nr, d] fp32: expert centroids e_i
 *   bias       device [Nr] fp32: routing bias b_i (read only here)
 *   topk_idx   device [T, K] int32 out: selected experts of each token,
 *              ordered by s+b descending; an exact tie goes to the lower index
 *   topk_gate  device [T, K] fp32 out: g = s / (sum of the selected s) -
 *              the gate keeps s, the bias only steers the selection
 *   topk_score device [T, K] fp32 out, may be NULL: s of the selected experts
 *   expert_load device [Nr] int32 out: number of tokens that selected each
 *              expert (overwritten, not accumulated)
 *   ws         device workspace of at least moe_route_workspace_bytes(T, d, Nr)
 *   Affinities are computed in fp32 (products exact, fp32 accumulation in
 *   blocks) and the sigmoid in fp32.
 *   Errors: MOE_EINVAL for NULL required pointers, T < 0, d < 1,
 *   Nr outside [1, MOE_MAX_EXPERTS], K outside [1, min(Nr, MOE_MAX_K)],
 *   d not a multiple of 8; MOE_EWORKSPACE when ws_bytes is too small.
 *   T == 0 is valid: expert_load is zeroed and nothing else is written.
 * ---------------------------------------------------------------------- */
size_t moe_route_workspace_bytes(int T, int d, int Nr);
moe_status moe_route(const void* u, moe_dtype u_t, const float* centroids, const float* bias,
                     int T, int d, int Nr, int K,
                     int32_t* topk_idx, float* topk_gate, float* topk_score, int32_t* expert_load,
                     void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_permute: expert-contiguous, padded row layout (stable counting sort).
 * Realises the per-expert token sets that the combine equation sums over;
 * no token is dropped (blog "DeepSeek 알고 아는 척 좀 해보자 – 단편: 671B
 * 파라미터의 괴물, DeepSeek-V3", section "DeepSeekMoE & load balancing").
 *
 * Segment i < Nr holds the rows (t, k) with topk_idx[t, k] == i in increasing
 * t; segment Nr + j (j < Ns) holds every token 0..T-1 in order (shared expert
 * j, gate 1).  Each segment is padded with rows of token -1 to a multiple of
 * tile_m (a power of two in [1, MOE_TILE_ROWS]).
 *
 *   topk_idx   device [T, K] int32 in (from moe_route)
 *   seg_offset device [Nr+Ns+1] int32 out: first row of each segment;
 *              seg_offset[Nr+Ns] = padded rows in use
 *   row_token  device [P_max] int32 out: token of every row, -1 = padding
 *              (rows from seg_offset[Nr+Ns] to P_max are -1 as well)
 *   inv_row    device [T, K] int32 out: row that holds (t, k)
 *   tile_map   device [tiles_max, 4] int32 out: in segment order, each
 *              segment cut into tiles of MOE_TILE_ROWS rows (the last one
 *              shorter): {segment, first row, rows, token rows}; the token
 *              rows of a tile come first, its padding rows after them
 *   n_tiles    device [1] int32 out: entries of tile_map in use
 *   P_max = moe_permute_rows(...), tiles_max = moe_permute_tiles_max(...)
 *   Errors: MOE_EINVAL for NULL pointers, bad sizes or tile_m;
 *   MOE_EWORKSPACE when ws_bytes < moe_permute_workspace_bytes(...).
 * ---------------------------------------------------------------------- */
size_t moe_permute_rows(int T, int K, int Nr, int Ns, int tile_m);
size_t moe_permute_tiles_max(int T, int K, int Nr, int Ns, int tile_m);
size_t moe_permute_workspace_bytes(int T, int K, int Nr, int Ns);
moe_status moe_permute(const int32_t* topk_idx, int T, int K, int Nr, int Ns, int tile_m,
                       int32_t* seg_offset, int32_t* row_token, int32_t* inv_row,
                       int32_t* tile_map, int32_t* n_tiles,
                       void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_permute_noalloc: moe_permute without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  It allocates nothing:
 * the same kernels use a 4 MiB device array of the library's own (one copy
 * per GPU, held until the process ends; its address is looked up once per
 * device on the first call made with that device current).  Results are
 * those of moe_permute, bit for bit.
 *   Arguments, layouts and errors as moe_permute, without ws / ws_bytes;
 *   MOE_EWORKSPACE when the sizes need more than the array holds:
 *   moe_permute_workspace_bytes(T, K, Nr, Ns) must not exceed
 *   moe_permute_noalloc_scratch_bytes() (4 MiB: e.g. T up to 1048576 tokens
 *   with Nr = 256, T up to 262144 with Nr = 1024).
 *   Every call on one GPU uses that GPU's array: calls that overlap in time
 *   on one GPU (different streams or threads) race and must be serialised
 *   by the caller.
 * ---------------------------------------------------------------------- */
size_t moe_permute_noalloc_scratch_bytes(void);
moe_status moe_permute_noalloc(const int32_t* topk_idx, int T, int K, int Nr, int Ns, int tile_m,
                               int32_t* seg_offset, int32_t* row_token, int32_t* inv_row,
                               int32_t* tile_map, int32_t* n_tiles, void* stream);

/* ------------------------------------------------------------------------
 * moe_expert_gemm: every expert's SwiGLU FFN on its rows of the layout.
 * FFN^(s)_j and FFN^(r)_i of the [RG-MoE] combine equation; the pages do not
 * print the FFN form, this library uses SwiGLU:
 *   FFN(x) = W2 (SiLU(W_gate x) * (W_up x)),  SiLU(a) = a * sigmoid(a).
 * y[row] = FFN_{segment(row)}(x[row_token[row]]) for every token row of
 * every tile; padding rows of y (and of h in ws) may be left unwritten.
 *
 *   x, x_t      device [T, d]: MOE_F32, MOE_BF16, or MOE_E4M3 codes
 *   x_scale     device [T, d/128] fp32 for x_t == MOE_E4M3 (1x128 tiles,
 *               from fp8_quantize_tiles), else NULL
 *   w_t         MOE_F32, MOE_BF16 or MOE_E4M3 (128x128 blocks, [RG-FP8])
 *   w13         device [Nr+Ns, 2I, d]: rows 0..I-1 W_gate, rows I..2I-1 W_up
 *   w13_scale   device [Nr+Ns, 2I/128, d/128] fp32 for MOE_E4M3, else NULL
 *   w2          device [Nr+Ns, d, I]: W_down
 *   w2_scale    device [Nr+Ns, d/128, I/128] fp32 for MOE_E4M3, else NULL
 *   seg_offset, row_token, tile_map, n_tiles: from moe_permute
 *   ws          device workspace, moe_gemm_workspace_bytes(...) bytes: holds
 *               the hidden state h of every row
 *   y, y_t      device [P_max, d] out, MOE_F32 or MOE_BF16
 * Supported (x_t, w_t, y_t): (F32, F32, F32); (BF16, BF16, BF16|F32);
 * (BF16, E4M3, BF16) - fp8 weights, bf16 activations, h kept in bf16;
 * (E4M3, E4M3, BF16|F32) - fp8 activations and weights; h is re-quantised
 * to E4M3 in 1x128 tiles (scale rule of fp8_quantize_tiles) before the down
 * projection.
 * E4M3 scales must be powers of two, as fp8_quantize_tiles writes them: the
 * matrix instructions apply them as exponents per 128-wide K block, which is
 * exact; only the exponent field of a scale is read.  Accumulation is fp32
 * throughout.
 *   T == 0 is valid (x and x_scale may then be NULL): nothing is written.
 *   Errors: MOE_EINVAL for NULL pointers or bad sizes; MOE_EUNSUPPORTED for
 *   other dtype combinations; bf16 with d % 128 or I % 64 nonzero; E4M3 x E4M3
 *   with d or I not a multiple of 256 or above 8192; an operand of 2 GiB or
 *   more on the MFMA paths; MOE_EWORKSPACE for a small ws.
 * ---------------------------------------------------------------------- */
size_t moe_gemm_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m,
                                moe_dtype x_t, moe_dtype w_t);
moe_status moe_expert_gemm(const void* x, moe_dtype x_t, const float* x_scale,
                           moe_dtype w_t, const void* w13, const float* w13_scale,
                           const void* w2, const float* w2_scale,
                           int T, int K, int Nr, int Ns, int d, int I, int tile_m,
                           const int32_t* seg_offset, const int32_t* row_token,
                           const int32_t* tile_map, const int32_t* n_tiles,
                           void* ws, size_t ws_bytes,
                           void* y, moe_dtype y_t, void* stream);

/* ------------------------------------------------------------------------
 * moe_combine: h'_t = u_t + sum_j y[shared_j(t)] + sum_k g[t,k] y[inv_row[t,k]]
 * ([RG-MoE] combine equation).  Accumulates in fp32 in a fixed order
 * (residual, shared experts ascending, routed k ascending), so results are
 * bitwise reproducible.
 *
 *   u, u_t       device [T, d], MOE_F32 or MOE_BF16
 *   y, y_t       device [P_max, d] from moe_expert_gemm
 *   inv_row      device [T, K] int32, topk_gate device [T, K] fp32
 *   seg_offset   device [Nr+Ns+1] int32 (shared rows: seg_offset[Nr+j] + t)
 *   flags        MOE_COMBINE_* bits to drop terms
 *   out, out_t   device [T, d] out, MOE_F32 or MOE_BF16 (may not alias y)
 *   Errors: MOE_EINVAL for NULL pointers, bad sizes, d not a multiple of 8.
 * ---------------------------------------------------------------------- */
moe_status moe_combine(const void* u, moe_dtype u_t, const void* y, moe_dtype y_t,
                       const int32_t* inv_row, const float* topk_gate, const int32_t* seg_offset,
                       int T, int d, int K, int Nr, int Ns, unsigned flags,
                       void* out, moe_dtype out_t, void* stream);

/* ------------------------------------------------------------------------
 * moe_expert_gemm_combine: moe_expert_gemm and moe_combine in one call, the
 * combine fused into the down projection ([RG-MoE] combine equation):
 *   out[t] = u_t + sum_j y[shared_j(t)] + sum_k g[t,k] y[inv_row[t,k]]
 * with every y row added to its token's row of out by fp32 atomic adds in
 * the down projection's epilogue, so y is never written to memory (about
 * 2 GB less traffic per 8192-token V3 prefill step than moe_expert_gemm +
 * moe_combine).  The order of the adds is not fixed: results agree with
 * moe_combine's to fp32 rounding of the sum and are not bitwise
 * reproducible (use moe_combine for that).  y rows are summed unrounded
 * (moe_combine reads them rounded to y_t).
 *   Arguments as moe_expert_gemm (x, weights, layout, tile_m), plus
 *   inv_row, topk_gate device [T, K] from moe_permute / moe_route
 *   u, u_t       device [T, d] tokens, MOE_F32 or MOE_BF16 (the residual)
 *   flags        MOE_COMBINE_* bits, as moe_combine
 *   ws           device, moe_gemm_combine_workspace_bytes(...) bytes
 *   out          device [T, d] fp32 out (overwritten; may not alias u)
 *   Supported (x_t, w_t): (BF16, BF16) with d % 256 == 0 and I % 128 == 0;
 *   (E4M3, E4M3) with d, I multiples of 256 up to 8192; else
 *   MOE_EUNSUPPORTED.  Other errors as moe_expert_gemm and moe_combine.
 * ---------------------------------------------------------------------- */
size_t moe_gemm_combine_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m,
                                        moe_dtype x_t, moe_dtype w_t);
moe_status moe_expert_gemm_combine(const void* x, moe_dtype x_t, const float* x_scale,
                                   moe_dtype w_t, const void* w13, const float* w13_scale,
                                   const void* w2, const float* w2_scale,
                                   int T, int K, int Nr, int Ns, int d, int I, int tile_m,
                                   const int32_t* seg_offset, const int32_t* row_token,
                                   const int32_t* tile_map, const int32_t* n_tiles,
                                   const int32_t* inv_row, const float* topk_gate,
                                   const void* u, moe_dtype u_t, unsigned flags,
                                   void* ws, size_t ws_bytes, float* out, void* stream);

/* ------------------------------------------------------------------------
 * moe_bias_update: end-of-step bias rule ([RG-MoE] bias rule).  The pages do
 * not define "overloaded"; this library compares the load with the mean
 * load T*K/Nr exactly in integers: Nr*c_i > T*K -> b_i -= gamma,
 * Nr*c_i < T*K -> b_i += gamma, equal -> unchanged; one fp32 add.
 *
 *   expert_load  device [Nr] int32 (from moe_route of this step)
 *   total_assign T*K, the number of (token, expert) assignments of the step
 *   gamma        bias step (0.001 on the pages)
 *   bias         device [Nr] fp32, updated in place
 *   Errors: MOE_EINVAL for NULL pointers, Nr out of range, total_assign < 0,
 *   non-finite or negative gamma.
 * ---------------------------------------------------------------------- */
moe_status moe_bias_update(const int32_t* expert_load, int Nr, long long total_assign,
                           float gamma, float* bias, void* stream);

/* ------------------------------------------------------------------------
 * fp8_quantize_tiles: tile-wise E4M3 quantisation ([RG-FP8]: 1x128 tiles for
 * activations, 128x128 blocks for weights).  The pages give no scale rule;
 * this library uses, per tile, the power of two sc = 2^k with the smallest
 * k >= -126 such that amax <= 448 * sc (sc = 1 for an all-zero tile), and
 * code = round-to-nearest-even(x / sc) (exact division).  A power-of-two
 * scale is the E8M0 block scale the gfx950 scaled MFMA applies in hardware;
 * code * sc is exact in fp32 and in bf16.  NaN is never produced for finite
 * input.  Scales are stored as fp32 values.
 *
 *   x, x_t     device [rows, cols], MOE_F32 or MOE_BF16
 *   tile_rows  1 or 128 (rows must be a multiple of it); tile_cols 128
 *              (cols must be a multiple of it)
 *   q          device [rows, cols] uint8 out (E4M3 codes)
 *   scale      device [rows/tile_rows, cols/tile_cols] fp32 out
 *   Errors: MOE_EINVAL for NULL pointers, bad sizes or tile shapes.
 * ---------------------------------------------------------------------- */
moe_status fp8_quantize_tiles(const void* x, moe_dtype x_t, long long rows, long long cols,
                              int tile_rows, int tile_cols, uint8_t* q, float* scale, void* stream);

/* ------------------------------------------------------------------------
 * fp8_dequantize_tiles: the values that E4M3 tiles stand for ([RG-FP8]
 * tiles), out[r, c] = decode(q[r, c]) * scale[r / tile_rows, c / 128]: the
 * operand an E4M3 product multiplies.  With power-of-two scales (as
 * fp8_quantize_tiles writes them) every value is exact in fp32, and in bf16
 * for scales >= 2^-124.  The E4M3 training step uses it for Q(u), the input
 * its gate/up weight gradient takes (straight-through quantisers).
 *
 *   q          device [rows, cols] uint8 E4M3 codes
 *   scale      device [rows/tile_rows, cols/128] fp32
 *   tile_rows  1 or 128; tile_cols 128 (as fp8_quantize_tiles)
 *   out, out_t device [rows, cols] out, MOE_F32 or MOE_BF16
 *   Errors: MOE_EINVAL for NULL pointers, bad sizes or tile shapes, out_t.
 * ---------------------------------------------------------------------- */
moe_status fp8_dequantize_tiles(const uint8_t* q, const float* scale, long long rows, long long cols,
                                int tile_rows, int tile_cols, void* out, moe_dtype out_t, void* stream);

/* ------------------------------------------------------------------------
 * fp8_quantize_runs: E4M3 along the rows of the permuted layout, the token
 * axis along which a weight gradient sums ([RG-FP8] gives E4M3 for all
 * tensors but no tile along the tokens; the reading kept here is its 1x128
 * activation tile turned along that axis).  Segment e, rows
 * seg_offset[e] .. seg_offset[e+1]-1 (bounds clamped to [0, P]), is cut
 * into runs of 128 rows from its first row, the last run shorter; each
 * column of each run gets its own power-of-two scale by the rule of
 * fp8_quantize_tiles.  Run r of segment e is scale row run_offset[e] + r.
 *
 *   x, x_t     device, MOE_F32 or MOE_BF16: gather == 0: [P, cols], row r
 *              of the layout is x row r; gather != 0: [x_rows, cols], row r
 *              is x row row_token[r] (the token rows of moe_permute)
 *   row_token  device [P]: a row with row_token < 0 (padding), or whose
 *              token is not a row of x, counts as zeros
 *   seg_offset device [n_seg + 1] (moe_permute's, n_seg = Nr + Ns)
 *   run_offset device [n_seg + 1] int32 out: run_offset[e] = sum over
 *              e' < e of ceil(rows of e' / 128), run_offset[n_seg] = runs
 *   q          device [P, cols] uint8 out: codes of the rows of every
 *              segment (0 on padding rows); other rows untouched
 *   scale      device [fp8_quantize_runs_max(P, n_seg), cols] fp32 out:
 *              rows 0 .. runs-1 written
 *   Errors: MOE_EINVAL for NULL pointers (x may be NULL when it has no
 *   rows to read: P == 0, or gather with x_rows == 0), bad sizes
 *   (cols % 128 != 0, P < 0, n_seg < 1, gather == 0 with x_rows < P), x_t;
 *   MOE_EUNSUPPORTED for an operand of 2 GiB or more.
 * ---------------------------------------------------------------------- */
long long fp8_quantize_runs_max(long long P, int n_seg);  /* (P + 127 n_seg) / 128 */
moe_status fp8_quantize_runs(const void* x, moe_dtype x_t, long long x_rows, int cols,
                             const int32_t* row_token, int gather, const int32_t* seg_offset,
                             int n_seg, long long P, int32_t* run_offset, uint8_t* q,
                             float* scale, void* stream);

/* ========================================================================
 * Backward pass (bf16 activations and weights).  The pages print no
 * backward pass; these calls compute the chain rule through the forward
 * above.  The top-K selection and the bias b are piecewise constant in the
 * inputs, so no gradient flows through them and b receives none; the
 * gradient reaches the affinities only through the gates of the selected
 * experts.  With G = dL/dh' (the gradient of the layer output), one step is
 *   moe_expert_gemm_train (forward, keeping h and [a | b])
 *   moe_combine_backward  -> dy (gradient of every expert row), dgate, dz
 *   moe_expert_gemm_backward -> dx (gradient of every expert row's input),
 *                               dW13, dW2
 *   moe_route_backward    -> du, de
 * after moe_route / moe_permute of the forward (same buffers).
 * ====================================================================== */

/* ------------------------------------------------------------------------
 * moe_expert_gemm_train: moe_expert_gemm for (x_t, w_t) = (BF16, BF16) that
 * also keeps what the backward needs: h [P_max, I] (bf16, SiLU(a) * b) and
 * ab [P_max, 2I] (bf16: columns 0..I-1 a = W_gate x, I..2I-1 b = W_up x) of
 * every token row (padding rows unwritten).  y as in moe_expert_gemm.
 *   ws  device, moe_gemm_train_workspace_bytes(...) bytes (work schedule)
 *   Errors: as moe_expert_gemm; MOE_EUNSUPPORTED unless d % 256 == 0,
 *   I % 128 == 0 (d <= 65280, I <= 32640) and every operand < 2 GiB.
 * ---------------------------------------------------------------------- */
size_t moe_gemm_train_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m);
moe_status moe_expert_gemm_train(const void* x, const void* w13, const void* w2,
                                 int T, int K, int Nr, int Ns, int d, int I, int tile_m,
                                 const int32_t* seg_offset, const int32_t* row_token,
                                 const int32_t* tile_map, const int32_t* n_tiles,
                                 void* ws, size_t ws_bytes, void* h, void* ab,
                                 void* y, moe_dtype y_t, void* stream);

/* ------------------------------------------------------------------------
 * moe_expert_gemm_train_w8: moe_expert_gemm for (x_t, w_t) = (E4M3, E4M3)
 * ([RG-FP8]: x in 1x128 tiles, weights in 128x128 blocks, h re-quantised in
 * 1x128 tiles before the down projection) that also keeps, for
 * moe_expert_gemm_backward_w8, ab [P_max, 2I] (bf16 pre-activations from
 * the fp32 accumulators) and h [P_max, I] (bf16: the E4M3 h that the down
 * projection multiplies, code x scale, exact).  y as in moe_expert_gemm.
 *   x, x_scale     device [T, d] E4M3 codes, [T, d/128] fp32 scales
 *   w13 .. w2_scale as moe_expert_gemm_backward_w8
 *   ws  device, moe_gemm_train_w8_workspace_bytes(...) bytes (work schedule
 *       and the E4M3 h)
 *   Errors: as moe_expert_gemm_train; MOE_EUNSUPPORTED unless d % 256 == 0,
 *   I % 256 == 0, d <= 8192 and I <= 8192.
 * ---------------------------------------------------------------------- */
size_t moe_gemm_train_w8_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m);
moe_status moe_expert_gemm_train_w8(const uint8_t* x, const float* x_scale,
                                    const uint8_t* w13, const float* w13_scale,
                                    const uint8_t* w2, const float* w2_scale,
                                    int T, int K, int Nr, int Ns, int d, int I, int tile_m,
                                    const int32_t* seg_offset, const int32_t* row_token,
                                    const int32_t* tile_map, const int32_t* n_tiles,
                                    void* ws, size_t ws_bytes, void* h, void* ab,
                                    void* y, moe_dtype y_t, void* stream);

/* ------------------------------------------------------------------------
 * moe_combine_backward: gradients of the [RG-MoE] combine equation and of
 * the gate equation (g = s / sum of the selected s) for one step.
 *   grad_out, g_t  device [T, d] G = dL/dh', MOE_F32 or MOE_BF16
 *   y, y_t         device [P_max, d] expert outputs of the forward
 *   inv_row, topk_gate, topk_score: device [T, K] from moe_permute/moe_route
 *   seg_offset     device [Nr+Ns+1]
 *   dy             device [P_max, d] bf16 out: g[t,k] * G_t on row (t, k),
 *                  G_t on the shared rows of t (padding rows unwritten)
 *   dgate          device [T, K] fp32 out: <G_t, y[row(t, k)]>
 *   dz             device [T, K] fp32 out: dL/d(u_t . e_i) of the selected
 *                  experts, (dgate_k - sum_j g_j dgate_j) / S_t * s (1 - s)
 *   dz_row         device [P_max] fp32 out: dz of row (t, k) at that row
 * The dot products are summed in fp32 in a fixed order (deterministic).
 *   Errors: MOE_EINVAL for NULL pointers, bad sizes, d % 8 != 0.
 * ---------------------------------------------------------------------- */
moe_status moe_combine_backward(const void* grad_out, moe_dtype g_t, const void* y, moe_dtype y_t,
                                const int32_t* inv_row, const float* topk_gate, const float* topk_score,
                                const int32_t* seg_offset, int T, int d, int K, int Nr, int Ns,
                                void* dy, float* dgate, float* dz, float* dz_row, void* stream);

/* ------------------------------------------------------------------------
 * moe_expert_gemm_backward: gradients of every expert's SwiGLU FFN on its
 * rows (bf16 operands, fp32 accumulation on the matrix cores):
 *   dh = dy W2,  da = dh * b * SiLU'(a),  db = dh * SiLU(a)
 *   dx = [da | db] W13 (per row),  dW2_e = sum_rows dy^T h,
 *   dW13_e = sum_rows [da | db]^T x
 *   x              device [T, d] bf16 tokens of the forward
 *   w13, w2        device bf16 weights as in moe_expert_gemm
 *   h, ab          device, from moe_expert_gemm_train
 *   dy             device [P_max, d] bf16 from moe_combine_backward
 *   ws             device, moe_gemm_backward_workspace_bytes(...) bytes
 *                  (holds [da | db] of every row and the weight-gradient
 *                  kernels' list of experts per XCD)
 *   dx             device [P_max, d] bf16 out (padding rows unwritten)
 *   dw13, dw2      device [Nr+Ns, 2I, d] and [Nr+Ns, d, I] out (overwritten;
 *                  experts with no rows get zeros), dw_t MOE_F32 or MOE_BF16
 * Every output element is summed by one thread in a fixed order.
 *   Errors: MOE_EINVAL for NULL pointers or bad sizes; MOE_EUNSUPPORTED
 *   unless d % 256 == 0, I % 128 == 0 and every operand < 2 GiB;
 *   MOE_EWORKSPACE for a small ws.
 * ---------------------------------------------------------------------- */
size_t moe_gemm_backward_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m);
moe_status moe_expert_gemm_backward(const void* x, const void* w13, const void* w2,
                                    const void* h, const void* ab, const void* dy,
                                    int T, int K, int Nr, int Ns, int d, int I, int tile_m,
                                    const int32_t* seg_offset, const int32_t* row_token,
                                    const int32_t* tile_map, const int32_t* n_tiles,
                                    void* ws, size_t ws_bytes, void* dx,
                                    void* dw13, void* dw2, moe_dtype dw_t, void* stream);

/* ------------------------------------------------------------------------
 * moe_expert_gemm_backward_w8: moe_expert_gemm_backward with the two
 * input-gradient products on E4M3 operands, after [RG-FP8] (E4M3
 * everywhere, 1x128 tiles for activations, 128x128 blocks for weights):
 * dy and then [da | db] are quantised in 1x128
 * tiles along their K axis (d, 2I) with power-of-two scales, and multiply
 * the E4M3 weights of the forward, block-scaled E8M0 on the matrix cores:
 *   dh = Q(dy) Q(W2),  dx = Q([da | db]) Q(W13)
 * The weight gradients are those of moe_expert_gemm_backward (bf16 dy,
 * [da | db], h, x): their K axis is the token axis, for which the pages give
 * no tiling.  x is the expert input as the forward multiplied it: the bf16
 * u after a bf16 forward; after the E4M3 forward (moe_expert_gemm_train_w8)
 * Q(u) decoded by fp8_dequantize_tiles, so that dW13 = [da | db]^T Q(u) is
 * the gradient through a straight-through quantiser.  Codes of dy and
 * [da | db] are decided from their bf16 values.
 *   w13, w13_scale device E4M3 [Nr+Ns, 2I, d] with fp32 [Nr+Ns, 2I/128,
 *                  d/128] block scales, w2, w2_scale [Nr+Ns, d, I] with
 *                  [Nr+Ns, d/128, I/128] (as fp8_quantize_tiles writes them
 *                  with 128x128 tiles; powers of two)
 *   ws             device, moe_gemm_backward_w8_workspace_bytes(...) bytes
 *   every other argument as moe_expert_gemm_backward
 *   Errors: as moe_expert_gemm_backward; MOE_EUNSUPPORTED also for
 *   d > 16384 or I > 8192.
 * ---------------------------------------------------------------------- */
size_t moe_gemm_backward_w8_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m);
moe_status moe_expert_gemm_backward_w8(const void* x, const uint8_t* w13, const float* w13_scale,
                                       const uint8_t* w2, const float* w2_scale,
                                       const void* h, const void* ab, const void* dy,
                                       int T, int K, int Nr, int Ns, int d, int I, int tile_m,
                                       const int32_t* seg_offset, const int32_t* row_token,
                                       const int32_t* tile_map, const int32_t* n_tiles,
                                       void* ws, size_t ws_bytes, void* dx,
                                       void* dw13, void* dw2, moe_dtype dw_t, void* stream);

/* ------------------------------------------------------------------------
 * moe_expert_gemm_backward_f8: moe_expert_gemm_backward_w8 with the two
 * weight-gradient products on E4M3 operands too, so that every product of
 * the backward is E4M3 ([RG-FP8]: E4M3 for all tensors).  Their K axis is
 * the token axis: both operands are quantised in runs of 128 rows of one
 * expert per column (fp8_quantize_runs), each run and column with its
 * power-of-two scale, and multiply on the block-scaled matrix cores:
 *   dW2_e  = R(dy_e)^T R(h_e),  dW13_e = R([da | db]_e)^T R(x_e)
 * (fp32 accumulation).  dy and [da | db] are quantised from their bf16
 * values; h and x are the bf16 operands of the forward (after the E4M3
 * forward: the decoded E4M3 h and Q(u), exact in bf16), quantised again
 * along the tokens.  dx as in moe_expert_gemm_backward_w8.  dy and
 * [da | db] are each read once for both of their E4M3 layouts (the 1x128
 * tiles of the input-gradient products and the token runs).
 *   ws  device, moe_gemm_backward_f8_workspace_bytes(...) bytes
 *   every other argument as moe_expert_gemm_backward_w8
 *   Errors: as moe_expert_gemm_backward_w8.
 * ---------------------------------------------------------------------- */
size_t moe_gemm_backward_f8_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m);
moe_status moe_expert_gemm_backward_f8(const void* x, const uint8_t* w13, const float* w13_scale,
                                       const uint8_t* w2, const float* w2_scale,
                                       const void* h, const void* ab, const void* dy,
                                       int T, int K, int Nr, int Ns, int d, int I, int tile_m,
                                       const int32_t* seg_offset, const int32_t* row_token,
                                       const int32_t* tile_map, const int32_t* n_tiles,
                                       void* ws, size_t ws_bytes, void* dx,
                                       void* dw13, void* dw2, moe_dtype dw_t, void* stream);

/* ------------------------------------------------------------------------
 * moe_route_backward: the layer's input and centroid gradients.
 *   du_t = G_t + sum of dx over the token's shared and routed rows
 *          + sum_k dz[t,k] e_{topk_idx[t,k]}           (fp32, that order)
 *   de_i = sum over the rows of segment i, in row order, of dz_row * u_t
 *   grad_out, g_t  device [T, d] G, MOE_F32 or MOE_BF16
 *   dx             device [P_max, d] bf16 from moe_expert_gemm_backward
 *   u, u_t         device [T, d] tokens, MOE_F32 or MOE_BF16
 *   centroids      device [Nr, d] fp32
 *   topk_idx, inv_row, dz: device [T, K]; dz_row device [P_max]
 *   seg_offset, row_token: from moe_permute
 *   du, du_t       device [T, d] out, MOE_F32 or MOE_BF16
 *   de             device [Nr, d] fp32 out (overwritten)
 *   Errors: MOE_EINVAL for NULL pointers, bad sizes, d % 8 != 0.
 * ---------------------------------------------------------------------- */
moe_status moe_route_backward(const void* grad_out, moe_dtype g_t, const void* dx,
                              const void* u, moe_dtype u_t, const float* centroids,
                              const int32_t* topk_idx, const int32_t* inv_row,
                              const float* dz, const float* dz_row,
                              const int32_t* seg_offset, const int32_t* row_token,
                              int T, int d, int K, int Nr, int Ns,
                              void* du, moe_dtype du_t, float* de, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
