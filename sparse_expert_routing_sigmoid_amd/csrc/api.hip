// extern "C" entry points of libmoe_mi355x: argument checks, workspace
// bookkeeping and dispatch to the kernels.  See include/moe_mi355x.h for the
// contract of every call.
#include "common.h"

namespace moe {

// Kernel-side entry points (defined in the other translation units).
size_t route_workspace_bytes(int T, int d, int Nr);
moe_status route(const void* u, moe_dtype u_t, const float* centroids, const float* bias, int T, int d, int Nr, int K,
                 int32_t* topk_idx, float* topk_gate, float* topk_score, int32_t* expert_load, void* ws,
                 size_t ws_bytes, void* stream);
size_t permute_rows(int T, int K, int Nr, int Ns, int tile_m);
size_t permute_tiles_max(int T, int K, int Nr, int Ns, int tile_m);
size_t permute_workspace_bytes(int T, int K, int Nr, int Ns);
moe_status permute(const int32_t* topk_idx, int T, int K, int Nr, int Ns, int tile_m, int32_t* seg_offset,
                   int32_t* row_token, int32_t* inv_row, int32_t* tile_map, int32_t* n_tiles, void* ws,
                   size_t ws_bytes, void* stream);
size_t permute_noalloc_scratch_bytes();
moe_status permute_noalloc(const int32_t* topk_idx, int T, int K, int Nr, int Ns, int tile_m, int32_t* seg_offset,
                           int32_t* row_token, int32_t* inv_row, int32_t* tile_map, int32_t* n_tiles, void* stream);
moe_status combine(const void* u, moe_dtype u_t, const void* y, moe_dtype y_t, const int32_t* inv_row,
                   const float* topk_gate, const int32_t* seg_offset, int T, int d, int K, int Nr, int Ns,
                   unsigned flags, void* out, moe_dtype out_t, void* stream);
moe_status bias_update(const int32_t* expert_load, int Nr, long long total_assign, float gamma, float* bias,
                       void* stream);
moe_status quantize_tiles(const void* x, moe_dtype x_t, long long rows, long long cols, int tile_rows, int tile_cols,
                          uint8_t* q, float* scale, void* stream);
moe_status dequantize_tiles(const uint8_t* q, const float* scale, long long rows, long long cols, int tile_rows,
                            int tile_cols, void* out, moe_dtype out_t, void* stream);
long long quantize_runs_max(long long P, int n_seg);
moe_status quantize_runs(const void* x, moe_dtype x_t, long long x_rows, int cols, const int32_t* row_token,
                         int gather, const int32_t* seg_offset, int n_seg, long long P, int32_t* run_offset,
                         uint8_t* q, float* scale, void* stream);
size_t gemm_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m, moe_dtype x_t, moe_dtype w_t);
moe_status expert_gemm(const void* x, moe_dtype x_t, const float* x_scale, moe_dtype w_t, const void* w13,
                       const float* w13_scale, const void* w2, const float* w2_scale, int T, int K, int Nr, int Ns,
                       int d, int I, int tile_m, const int32_t* seg_offset, const int32_t* row_token,
                       const int32_t* tile_map, const int32_t* n_tiles, void* ws, size_t ws_bytes, void* y,
                       moe_dtype y_t, void* stream);

size_t gemm_combine_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m, moe_dtype x_t,
                                    moe_dtype w_t);
moe_status expert_gemm_combine(const void* x, moe_dtype x_t, const float* x_scale, moe_dtype w_t, const void* w13,
                               const float* w13_scale, const void* w2, const float* w2_scale, int T, int K, int Nr,
                               int Ns, int d, int I, int tile_m, const int32_t* seg_offset, const int32_t* row_token,
                               const int32_t* tile_map, const int32_t* n_tiles, const int32_t* inv_row,
                               const float* topk_gate, const void* u, moe_dtype u_t, unsigned flags, void* ws,
                               size_t ws_bytes, float* out, void* stream);
size_t gemm_train_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m);
moe_status expert_gemm_train(const void* x, const void* w13, const void* w2, int T, int K, int Nr, int Ns, int d,
                             int I, int tile_m, const int32_t* seg_offset, const int32_t* row_token,
                             const int32_t* tile_map, const int32_t* n_tiles, void* ws, size_t ws_bytes, void* h,
                             void* ab, void* y, moe_dtype y_t, void* stream);
moe_status combine_backward(const void* grad_out, moe_dtype g_t, const void* y, moe_dtype y_t,
                            const int32_t* inv_row, const float* topk_gate, const float* topk_score,
                            const int32_t* seg_offset, int T, int d, int K, int Nr, int Ns, void* dy, float* dgate,
                            float* dz, float* dz_row, void* stream);
size_t gemm_backward_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m);
moe_status expert_gemm_backward(const void* x, const void* w13, const void* w2, const void* h, const void* ab,
                                const void* dy, int T, int K, int Nr, int Ns, int d, int I, int tile_m,
                                const int32_t* seg_offset, const int32_t* row_token, const int32_t* tile_map,
                                const int32_t* n_tiles, void* ws, size_t ws_bytes, void* dx, void* dw13, void* dw2,
                                moe_dtype dw_t, void* stream);
size_t gemm_train_w8_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m);
moe_status expert_gemm_train_w8(const uint8_t* x, const float* x_scale, const uint8_t* w13, const float* w13_scale,
                                const uint8_t* w2, const float* w2_scale, int T, int K, int Nr, int Ns, int d, int I,
                                int tile_m, const int32_t* seg_offset, const int32_t* row_token,
                                const int32_t* tile_map, const int32_t* n_tiles, void* ws, size_t ws_bytes, void* h,
                                void* ab, void* y, moe_dtype y_t, void* stream);
size_t gemm_backward_w8_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m);
moe_status expert_gemm_backward_w8(const void* x, const uint8_t* w13, const float* w13_scale, const uint8_t* w2,
                                   const float* w2_scale, const void* h, const void* ab, const void* dy, int T, int K,
                                   int Nr, int Ns, int d, int I, int tile_m, const int32_t* seg_offset,
                                   const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles,
                                   void* ws, size_t ws_bytes, void* dx, void* dw13, void* dw2, moe_dtype dw_t,
                                   void* stream);
size_t gemm_backward_f8_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m);
moe_status expert_gemm_backward_f8(const void* x, const uint8_t* w13, const float* w13_scale, const uint8_t* w2,
                                   const float* w2_scale, const void* h, const void* ab, const void* dy, int T, int K,
                                   int Nr, int Ns, int d, int I, int tile_m, const int32_t* seg_offset,
                                   const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles,
                                   void* ws, size_t ws_bytes, void* dx, void* dw13, void* dw2, moe_dtype dw_t,
                                   void* stream);
moe_status route_backward(const void* grad_out, moe_dtype g_t, const void* dx, const void* u, moe_dtype u_t,
                          const float* centroids, const int32_t* topk_idx, const int32_t* inv_row, const float* dz,
                          const float* dz_row, const int32_t* seg_offset, const int32_t* row_token, int T, int d,
                          int K, int Nr, int Ns, void* du, moe_dtype du_t, float* de, void* stream);

namespace {
thread_local std::string g_last_error;
}

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }

moe_status launch_status(const char* where) {
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error(std::string(where) + ": " + hipGetErrorString(err));
    return MOE_EHIP;
  }
  return MOE_OK;
}

}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE";
    case MOE_EHIP: return "MOE_EHIP";
    default: return "MOE_UNKNOWN";
  }
}

const char* moe_last_error(void) { return moe::g_last_error.c_str(); }

size_t moe_route_workspace_bytes(int T, int d, int Nr) { return moe::route_workspace_bytes(T, d, Nr); }

moe_status moe_route(const void* u, moe_dtype u_t, const float* centroids, const float* bias, int T, int d, int Nr,
                     int K, int32_t* topk_idx, float* topk_gate, float* topk_score, int32_t* expert_load, void* ws,
                     size_t ws_bytes, void* stream) {
  moe::clear_error();
  return moe::route(u, u_t, centroids, bias, T, d, Nr, K, topk_idx, topk_gate, topk_score, expert_load, ws, ws_bytes,
                    stream);
}

size_t moe_permute_rows(int T, int K, int Nr, int Ns, int tile_m) { return moe::permute_rows(T, K, Nr, Ns, tile_m); }
size_t moe_permute_tiles_max(int T, int K, int Nr, int Ns, int tile_m) {
  return moe::permute_tiles_max(T, K, Nr, Ns, tile_m);
}
size_t moe_permute_workspace_bytes(int T, int K, int Nr, int Ns) {
  return moe::permute_workspace_bytes(T, K, Nr, Ns);
}

moe_status moe_permute(const int32_t* topk_idx, int T, int K, int Nr, int Ns, int tile_m, int32_t* seg_offset,
                       int32_t* row_token, int32_t* inv_row, int32_t* tile_map, int32_t* n_tiles, void* ws,
                       size_t ws_bytes, void* stream) {
  moe::clear_error();
  return moe::permute(topk_idx, T, K, Nr, Ns, tile_m, seg_offset, row_token, inv_row, tile_map, n_tiles, ws, ws_bytes,
                      stream);
}

size_t moe_permute_noalloc_scratch_bytes(void) { return moe::permute_noalloc_scratch_bytes(); }

moe_status moe_permute_noalloc(const int32_t* topk_idx, int T, int K, int Nr, int Ns, int tile_m, int32_t* seg_offset,
                               int32_t* row_token, int32_t* inv_row, int32_t* tile_map, int32_t* n_tiles,
                               void* stream) {
  moe::clear_error();
  return moe::permute_noalloc(topk_idx, T, K, Nr, Ns, tile_m, seg_offset, row_token, inv_row, tile_map, n_tiles,
                              stream);
}

size_t moe_gemm_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m, moe_dtype x_t,
                                moe_dtype w_t) {
  return moe::gemm_workspace_bytes(T, K, Nr, Ns, d, I, tile_m, x_t, w_t);
}

moe_status moe_expert_gemm(const void* x, moe_dtype x_t, const float* x_scale, moe_dtype w_t, const void* w13,
                           const float* w13_scale, const void* w2, const float* w2_scale, int T, int K, int Nr,
                           int Ns, int d, int I, int tile_m, const int32_t* seg_offset, const int32_t* row_token,
                           const int32_t* tile_map, const int32_t* n_tiles, void* ws, size_t ws_bytes, void* y,
                           moe_dtype y_t, void* stream) {
  moe::clear_error();
  return moe::expert_gemm(x, x_t, x_scale, w_t, w13, w13_scale, w2, w2_scale, T, K, Nr, Ns, d, I, tile_m, seg_offset,
                          row_token, tile_map, n_tiles, ws, ws_bytes, y, y_t, stream);
}

size_t moe_gemm_combine_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m, moe_dtype x_t,
                                        moe_dtype w_t) {
  return moe::gemm_combine_workspace_bytes(T, K, Nr, Ns, d, I, tile_m, x_t, w_t);
}

moe_status moe_expert_gemm_combine(const void* x, moe_dtype x_t, const float* x_scale, moe_dtype w_t, const void* w13,
                                   const float* w13_scale, const void* w2, const float* w2_scale, int T, int K,
                                   int Nr, int Ns, int d, int I, int tile_m, const int32_t* seg_offset,
                                   const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles,
                                   const int32_t* inv_row, const float* topk_gate, const void* u, moe_dtype u_t,
                                   unsigned flags, void* ws, size_t ws_bytes, float* out, void* stream) {
  moe::clear_error();
  return moe::expert_gemm_combine(x, x_t, x_scale, w_t, w13, w13_scale, w2, w2_scale, T, K, Nr, Ns, d, I, tile_m,
                                  seg_offset, row_token, tile_map, n_tiles, inv_row, topk_gate, u, u_t, flags, ws,
                                  ws_bytes, out, stream);
}

moe_status moe_combine(const void* u, moe_dtype u_t, const void* y, moe_dtype y_t, const int32_t* inv_row,
                       const float* topk_gate, const int32_t* seg_offset, int T, int d, int K, int Nr, int Ns,
                       unsigned flags, void* out, moe_dtype out_t, void* stream) {
  moe::clear_error();
  return moe::combine(u, u_t, y, y_t, inv_row, topk_gate, seg_offset, T, d, K, Nr, Ns, flags, out, out_t, stream);
}

moe_status moe_bias_update(const int32_t* expert_load, int Nr, long long total_assign, float gamma, float* bias,
                           void* stream) {
  moe::clear_error();
  return moe::bias_update(expert_load, Nr, total_assign, gamma, bias, stream);
}

moe_status fp8_quantize_tiles(const void* x, moe_dtype x_t, long long rows, long long cols, int tile_rows,
                              int tile_cols, uint8_t* q, float* scale, void* stream) {
  moe::clear_error();
  return moe::quantize_tiles(x, x_t, rows, cols, tile_rows, tile_cols, q, scale, stream);
}

moe_status fp8_dequantize_tiles(const uint8_t* q, const float* scale, long long rows, long long cols, int tile_rows,
                                int tile_cols, void* out, moe_dtype out_t, void* stream) {
  moe::clear_error();
  return moe::dequantize_tiles(q, scale, rows, cols, tile_rows, tile_cols, out, out_t, stream);
}

long long fp8_quantize_runs_max(long long P, int n_seg) {
  return P < 0 || n_seg < 0 ? 0 : moe::quantize_runs_max(P, n_seg);
}

moe_status fp8_quantize_runs(const void* x, moe_dtype x_t, long long x_rows, int cols, const int32_t* row_token,
                             int gather, const int32_t* seg_offset, int n_seg, long long P, int32_t* run_offset,
                             uint8_t* q, float* scale, void* stream) {
  moe::clear_error();
  return moe::quantize_runs(x, x_t, x_rows, cols, row_token, gather, seg_offset, n_seg, P, run_offset, q, scale,
                            stream);
}

size_t moe_gemm_train_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  return moe::gemm_train_workspace_bytes(T, K, Nr, Ns, d, I, tile_m);
}

moe_status moe_expert_gemm_train(const void* x, const void* w13, const void* w2, int T, int K, int Nr, int Ns, int d,
                                 int I, int tile_m, const int32_t* seg_offset, const int32_t* row_token,
                                 const int32_t* tile_map, const int32_t* n_tiles, void* ws, size_t ws_bytes, void* h,
                                 void* ab, void* y, moe_dtype y_t, void* stream) {
  moe::clear_error();
  return moe::expert_gemm_train(x, w13, w2, T, K, Nr, Ns, d, I, tile_m, seg_offset, row_token, tile_map, n_tiles, ws,
                                ws_bytes, h, ab, y, y_t, stream);
}

moe_status moe_combine_backward(const void* grad_out, moe_dtype g_t, const void* y, moe_dtype y_t,
                                const int32_t* inv_row, const float* topk_gate, const float* topk_score,
                                const int32_t* seg_offset, int T, int d, int K, int Nr, int Ns, void* dy,
                                float* dgate, float* dz, float* dz_row, void* stream) {
  moe::clear_error();
  return moe::combine_backward(grad_out, g_t, y, y_t, inv_row, topk_gate, topk_score, seg_offset, T, d, K, Nr, Ns,
                               dy, dgate, dz, dz_row, stream);
}

size_t moe_gemm_backward_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  return moe::gemm_backward_workspace_bytes(T, K, Nr, Ns, d, I, tile_m);
}

moe_status moe_expert_gemm_backward(const void* x, const void* w13, const void* w2, const void* h, const void* ab,
                                    const void* dy, int T, int K, int Nr, int Ns, int d, int I, int tile_m,
                                    const int32_t* seg_offset, const int32_t* row_token, const int32_t* tile_map,
                                    const int32_t* n_tiles, void* ws, size_t ws_bytes, void* dx, void* dw13,
                                    void* dw2, moe_dtype dw_t, void* stream) {
  moe::clear_error();
  return moe::expert_gemm_backward(x, w13, w2, h, ab, dy, T, K, Nr, Ns, d, I, tile_m, seg_offset, row_token, tile_map,
                                   n_tiles, ws, ws_bytes, dx, dw13, dw2, dw_t, stream);
}

size_t moe_gemm_train_w8_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  return moe::gemm_train_w8_workspace_bytes(T, K, Nr, Ns, d, I, tile_m);
}

moe_status moe_expert_gemm_train_w8(const uint8_t* x, const float* x_scale, const uint8_t* w13,
                                    const float* w13_scale, const uint8_t* w2, const float* w2_scale, int T, int K,
                                    int Nr, int Ns, int d, int I, int tile_m, const int32_t* seg_offset,
                                    const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles,
                                    void* ws, size_t ws_bytes, void* h, void* ab, void* y, moe_dtype y_t,
                                    void* stream) {
  moe::clear_error();
  return moe::expert_gemm_train_w8(x, x_scale, w13, w13_scale, w2, w2_scale, T, K, Nr, Ns, d, I, tile_m, seg_offset,
                                   row_token, tile_map, n_tiles, ws, ws_bytes, h, ab, y, y_t, stream);
}

size_t moe_gemm_backward_w8_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  return moe::gemm_backward_w8_workspace_bytes(T, K, Nr, Ns, d, I, tile_m);
}

moe_status moe_expert_gemm_backward_w8(const void* x, const uint8_t* w13, const float* w13_scale, const uint8_t* w2,
                                       const float* w2_scale, const void* h, const void* ab, const void* dy, int T,
                                       int K, int Nr, int Ns, int d, int I, int tile_m, const int32_t* seg_offset,
                                       const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles,
                                       void* ws, size_t ws_bytes, void* dx, void* dw13, void* dw2, moe_dtype dw_t,
                                       void* stream) {
  moe::clear_error();
  return moe::expert_gemm_backward_w8(x, w13, w13_scale, w2, w2_scale, h, ab, dy, T, K, Nr, Ns, d, I, tile_m,
                                      seg_offset, row_token, tile_map, n_tiles, ws, ws_bytes, dx, dw13, dw2, dw_t,
                                      stream);
}

size_t moe_gemm_backward_f8_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  return moe::gemm_backward_f8_workspace_bytes(T, K, Nr, Ns, d, I, tile_m);
}

moe_status moe_expert_gemm_backward_f8(const void* x, const uint8_t* w13, const float* w13_scale, const uint8_t* w2,
                                       const float* w2_scale, const void* h, const void* ab, const void* dy, int T,
                                       int K, int Nr, int Ns, int d, int I, int tile_m, const int32_t* seg_offset,
                                       const int32_t* row_token, const int32_t* tile_map, const int32_t* n_tiles,
                                       void* ws, size_t ws_bytes, void* dx, void* dw13, void* dw2, moe_dtype dw_t,
                                       void* stream) {
  moe::clear_error();
  return moe::expert_gemm_backward_f8(x, w13, w13_scale, w2, w2_scale, h, ab, dy, T, K, Nr, Ns, d, I, tile_m,
                                      seg_offset, row_token, tile_map, n_tiles, ws, ws_bytes, dx, dw13, dw2, dw_t,
                                      stream);
}

moe_status moe_route_backward(const void* grad_out, moe_dtype g_t, const void* dx, const void* u, moe_dtype u_t,
                              const float* centroids, const int32_t* topk_idx, const int32_t* inv_row,
                              const float* dz, const float* dz_row, const int32_t* seg_offset,
                              const int32_t* row_token, int T, int d, int K, int Nr, int Ns, void* du,
                              moe_dtype du_t, float* de, void* stream) {
  moe::clear_error();
  return moe::route_backward(grad_out, g_t, dx, u, u_t, centroids, topk_idx, inv_row, dz, dz_row, seg_offset,
                             row_token, T, d, K, Nr, Ns, du, du_t, de, stream);
}

}  // extern "C"
