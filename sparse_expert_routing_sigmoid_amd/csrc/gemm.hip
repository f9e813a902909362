// moe_expert_gemm: argument checks, workspace layout and dispatch of the
// grouped SwiGLU expert GEMMs to the kernel family of each dtype combination.
#include "common.h"

namespace moe {

size_t permute_rows(int T, int K, int Nr, int Ns, int tile_m);
size_t permute_tiles_max(int T, int K, int Nr, int Ns, int tile_m);

void launch_ffn_bf16(const uint16_t* x, const uint16_t* w13, const uint16_t* w2, const int32_t* row_token,
                     const int32_t* tile_map, const int32_t* n_tiles, int tiles_max, int d, int I, uint16_t* h,
                     void* y, bool y_f32, hipStream_t st);
bool ffn_bf16_persistent_ok(int d, int I);
size_t ffn_schedule_bytes(long long tiles_cap, int ntA, int ntB);
int ffn_schedule_max_tiles();
void launch_ffn_bf16_persistent(const uint16_t* x, const uint16_t* w13, const uint16_t* w2, const int32_t* row_token,
                                const int32_t* tile_map, const int32_t* n_tiles, int T, long long P, int d, int I,
                                int Nr, int cap, uint16_t* h, uint16_t* ab, void* y, bool y_f32, int* sched,
                                hipStream_t st, const float* row_gate = nullptr);
bool ffn_fp8_persistent_ok(int d, int I);
void launch_ffn_fp8_persistent(const uint8_t* x, const float* x_scale, const uint8_t* w13, const float* w13_scale,
                               const uint8_t* w2, const float* w2_scale, const int32_t* row_token,
                               const int32_t* tile_map, const int32_t* n_tiles, int T, long long P, int d, int I,
                               int Nr, int cap, uint8_t* h, float* h_scale, void* y, bool y_f32, int* sched,
                               hipStream_t st, uint16_t* ab = nullptr, uint16_t* hb = nullptr,
                               const float* row_gate = nullptr);
bool ffn_w8a16_ok(int d, int I);
void launch_ffn_w8a16(const uint16_t* x, const uint8_t* w13, const float* w13_scale, const uint8_t* w2,
                      const float* w2_scale, const int32_t* row_token, const int32_t* tile_map,
                      const int32_t* n_tiles, int tiles_max, int T, long long P, int d, int I, uint16_t* h, void* y,
                      bool y_f32, hipStream_t st);
void launch_ffn_f32(const float* x, const float* w13, const float* w2, const int32_t* row_token,
                    const int32_t* tile_map, const int32_t* n_tiles, int tiles_max, int d, int I, float* h, float* y,
                    hipStream_t st);

void launch_fused_combine_prep(const void* u, moe_dtype u_t, const int32_t* inv_row, const float* topk_gate,
                               const int32_t* seg_offset, int T, int d, int K, int Nr, int Ns, unsigned flags,
                               float* out, float* row_gate, hipStream_t st);

namespace {

enum class Path { F32, BF16, W8A16, FP8, NONE };

Path path_of(moe_dtype x_t, moe_dtype w_t) {
  if (x_t == MOE_F32 && w_t == MOE_F32) return Path::F32;
  if (x_t == MOE_BF16 && w_t == MOE_BF16) return Path::BF16;
  if (x_t == MOE_BF16 && w_t == MOE_E4M3) return Path::W8A16;
  if (x_t == MOE_E4M3 && w_t == MOE_E4M3) return Path::FP8;
  return Path::NONE;
}

// Bytes of h per row for each path (fp8 keeps codes plus one fp32 scale per
// 128 columns).
size_t h_row_bytes(Path p, int I) {
  switch (p) {
    case Path::F32: return (size_t)I * 4;
    case Path::BF16:
    case Path::W8A16: return (size_t)I * 2;
    case Path::FP8: return (size_t)I + (size_t)(I / 128) * 4;
    default: return 0;
  }
}

}  // namespace

// Workspace: the work schedule of the persistent kernels (counters and item
// lists), then h.
size_t gemm_sched_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m) {
  return ffn_schedule_bytes((long long)permute_tiles_max(T, K, Nr, Ns, tile_m), (I + 127) / 128, (d + 255) / 256);
}

size_t gemm_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m, moe_dtype x_t, moe_dtype w_t) {
  const Path p = path_of(x_t, w_t);
  if (p == Path::NONE || T < 0 || I < 1 || d < 1) return 0;
  const size_t P = permute_rows(T, K, Nr, Ns, tile_m);
  return gemm_sched_bytes(T, K, Nr, Ns, d, I, tile_m) + P * h_row_bytes(p, I);
}

moe_status expert_gemm(const void* x, moe_dtype x_t, const float* x_scale, moe_dtype w_t, const void* w13,
                       const float* w13_scale, const void* w2, const float* w2_scale, int T, int K, int Nr, int Ns,
                       int d, int I, int tile_m, const int32_t* seg_offset, const int32_t* row_token,
                       const int32_t* tile_map, const int32_t* n_tiles, void* ws, size_t ws_bytes, void* y,
                       moe_dtype y_t, void* stream) {
  MOE_REQUIRE(T >= 0 && d >= 1 && I >= 1, MOE_EINVAL, "need T >= 0, d >= 1, I >= 1");
  MOE_REQUIRE(Nr >= 1 && Ns >= 0 && Nr + Ns <= MOE_MAX_EXPERTS, MOE_EINVAL, "expert counts out of range");
  MOE_REQUIRE(K >= 1 && K <= MOE_MAX_K && K <= Nr, MOE_EINVAL, "K out of range");
  MOE_REQUIRE(tile_m >= 1 && tile_m <= MOE_TILE_ROWS && (tile_m & (tile_m - 1)) == 0, MOE_EINVAL, "bad tile_m");
  MOE_REQUIRE(x_t == MOE_F32 || x_t == MOE_BF16 || x_t == MOE_E4M3, MOE_EINVAL, "bad x_t");
  MOE_REQUIRE(w_t == MOE_F32 || w_t == MOE_BF16 || w_t == MOE_E4M3, MOE_EINVAL, "bad w_t");
  MOE_REQUIRE(y_t == MOE_F32 || y_t == MOE_BF16, MOE_EINVAL, "bad y_t");
  MOE_REQUIRE(w13 && w2 && seg_offset && row_token && tile_map && n_tiles && y, MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(T == 0 || x, MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(aligned16(x) && aligned16(w13) && aligned16(w2) && aligned16(y) && aligned16(ws), MOE_EINVAL,
              "x, w13, w2, y and ws must be 16-byte aligned");
  const Path p = path_of(x_t, w_t);
  MOE_REQUIRE(p != Path::NONE, MOE_EUNSUPPORTED, "unsupported (x_t, w_t) combination");
  MOE_REQUIRE(w_t != MOE_E4M3 || (w13_scale && w2_scale), MOE_EINVAL, "E4M3 weights need block scales");
  MOE_REQUIRE(T == 0 || x_t != MOE_E4M3 || x_scale, MOE_EINVAL, "E4M3 activations need tile scales");
  MOE_REQUIRE(ws && ws_bytes >= gemm_workspace_bytes(T, K, Nr, Ns, d, I, tile_m, x_t, w_t), MOE_EWORKSPACE,
              "workspace smaller than moe_gemm_workspace_bytes");
  const size_t P = permute_rows(T, K, Nr, Ns, tile_m);
  MOE_REQUIRE(P < (1ull << 31), MOE_EINVAL, "too many rows");
  const int tiles_max = (int)permute_tiles_max(T, K, Nr, Ns, tile_m);
  hipStream_t st = as_stream(stream);
  if (T == 0) return MOE_OK;
  // Workspace: the work schedule, then h.
  int* ws_sched = static_cast<int*>(ws);
  uint8_t* ws_h = static_cast<uint8_t*>(ws) + gemm_sched_bytes(T, K, Nr, Ns, d, I, tile_m);
  const bool sched_fits = tiles_max <= ffn_schedule_max_tiles();
  switch (p) {
    case Path::F32:
      MOE_REQUIRE(y_t == MOE_F32, MOE_EUNSUPPORTED, "fp32 path writes fp32 y");
      launch_ffn_f32(static_cast<const float*>(x), static_cast<const float*>(w13), static_cast<const float*>(w2),
                     row_token, tile_map, n_tiles, tiles_max, d, I, reinterpret_cast<float*>(ws_h),
                     static_cast<float*>(y), st);
      break;
    case Path::BF16:
      MOE_REQUIRE(d % 128 == 0 && I % 64 == 0, MOE_EUNSUPPORTED, "bf16 path needs d % 128 == 0 and I % 64 == 0");
      if (ffn_bf16_persistent_ok(d, I) && sched_fits && (unsigned long long)T * d * 2 < (1ull << 31) &&
          (unsigned long long)P * I * 2 < (1ull << 31) && (unsigned long long)3 * I * d * 2 < (1ull << 31))
        launch_ffn_bf16_persistent(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w13),
                                   static_cast<const uint16_t*>(w2), row_token, tile_map, n_tiles, T, (long long)P, d,
                                   I, Nr, tiles_max, reinterpret_cast<uint16_t*>(ws_h), nullptr, y, y_t == MOE_F32,
                                   ws_sched, st);
      else
        launch_ffn_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w13),
                        static_cast<const uint16_t*>(w2), row_token, tile_map, n_tiles, tiles_max, d, I,
                        reinterpret_cast<uint16_t*>(ws_h), y, y_t == MOE_F32, st);
      break;
    case Path::FP8: {
      MOE_REQUIRE(ffn_fp8_persistent_ok(d, I), MOE_EUNSUPPORTED,
                  "fp8 path needs d % 256 == 0, I % 256 == 0, d <= 8192 and I <= 8192");
      MOE_REQUIRE((unsigned long long)T * d < (1ull << 31) && (unsigned long long)P * I < (1ull << 31) &&
                      (unsigned long long)3 * I * d < (1ull << 31),
                  MOE_EUNSUPPORTED, "fp8 path: operand larger than 2 GiB");
      MOE_REQUIRE(sched_fits, MOE_EUNSUPPORTED, "fp8 path: more GEMM tiles than the work schedule holds");
      // h: E4M3 codes [P, I], then their 1x128 tile scales [P, I / 128].
      uint8_t* h_codes = ws_h;
      float* h_scale = reinterpret_cast<float*>(ws_h + P * (size_t)I);
      launch_ffn_fp8_persistent(static_cast<const uint8_t*>(x), x_scale, static_cast<const uint8_t*>(w13), w13_scale,
                                static_cast<const uint8_t*>(w2), w2_scale, row_token, tile_map, n_tiles, T,
                                (long long)P, d, I, Nr, tiles_max, h_codes, h_scale, y, y_t == MOE_F32, ws_sched, st);
      break;
    }
    case Path::W8A16:
      MOE_REQUIRE(ffn_w8a16_ok(d, I), MOE_EUNSUPPORTED,
                  "bf16 x E4M3 path needs d % 256 == 0, I % 256 == 0, d <= 8192 and I <= 8192");
      MOE_REQUIRE((unsigned long long)T * d * 2 < (1ull << 31) && (unsigned long long)P * I * 2 < (1ull << 31) &&
                      (unsigned long long)2 * I * d < (1ull << 31),
                  MOE_EUNSUPPORTED, "bf16 x E4M3 path: operand larger than 2 GiB");
      launch_ffn_w8a16(static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(w13), w13_scale,
                       static_cast<const uint8_t*>(w2), w2_scale, row_token, tile_map, n_tiles, tiles_max, T,
                       (long long)P, d, I, reinterpret_cast<uint16_t*>(ws_h), y, y_t == MOE_F32, st);
      break;
    default:
      MOE_REQUIRE(false, MOE_EUNSUPPORTED, "unsupported (x_t, w_t) combination");
  }
  return launch_status("moe_expert_gemm");
}

// ---------------------------------------------------------- fused combine --
// Workspace: that of moe_expert_gemm, then the gate of every permuted row
// (fp32 [P_max]).
size_t gemm_combine_workspace_bytes(int T, int K, int Nr, int Ns, int d, int I, int tile_m, moe_dtype x_t,
                                    moe_dtype w_t) {
  const size_t g = gemm_workspace_bytes(T, K, Nr, Ns, d, I, tile_m, x_t, w_t);
  if (g == 0 && T > 0) return 0;
  return (g + 255) / 256 * 256 + permute_rows(T, K, Nr, Ns, tile_m) * 4;
}

moe_status expert_gemm_combine(const void* x, moe_dtype x_t, const float* x_scale, moe_dtype w_t, const void* w13,
                               const float* w13_scale, const void* w2, const float* w2_scale, int T, int K, int Nr,
                               int Ns, int d, int I, int tile_m, const int32_t* seg_offset, const int32_t* row_token,
                               const int32_t* tile_map, const int32_t* n_tiles, const int32_t* inv_row,
                               const float* topk_gate, const void* u, moe_dtype u_t, unsigned flags, void* ws,
                               size_t ws_bytes, float* out, void* stream) {
  MOE_REQUIRE(T >= 0 && d >= 1 && I >= 1, MOE_EINVAL, "need T >= 0, d >= 1, I >= 1");
  MOE_REQUIRE(Nr >= 1 && Ns >= 0 && Nr + Ns <= MOE_MAX_EXPERTS, MOE_EINVAL, "expert counts out of range");
  MOE_REQUIRE(K >= 1 && K <= MOE_MAX_K && K <= Nr, MOE_EINVAL, "K out of range");
  MOE_REQUIRE(tile_m >= 1 && tile_m <= MOE_TILE_ROWS && (tile_m & (tile_m - 1)) == 0, MOE_EINVAL, "bad tile_m");
  MOE_REQUIRE((flags & ~7u) == 0, MOE_EINVAL, "unknown flag bits");
  MOE_REQUIRE(u_t == MOE_F32 || u_t == MOE_BF16, MOE_EINVAL, "u_t must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(d % 8 == 0, MOE_EINVAL, "d must be a multiple of 8");
  MOE_REQUIRE(w13 && w2 && seg_offset && row_token && tile_map && n_tiles && out, MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(T == 0 || (x && u && inv_row && topk_gate), MOE_EINVAL, "NULL pointer");
  MOE_REQUIRE(static_cast<const void*>(out) != u, MOE_EINVAL, "out aliases u");
  MOE_REQUIRE(aligned16(x) && aligned16(w13) && aligned16(w2) && aligned16(u) && aligned16(out) && aligned16(ws),
              MOE_EINVAL, "x, w13, w2, u, out and ws must be 16-byte aligned");
  const Path p = path_of(x_t, w_t);
  MOE_REQUIRE(p == Path::BF16 || p == Path::FP8, MOE_EUNSUPPORTED,
              "the fused combine runs on the (BF16, BF16) and (E4M3, E4M3) persistent paths");
  MOE_REQUIRE(w_t != MOE_E4M3 || (w13_scale && w2_scale), MOE_EINVAL, "E4M3 weights need block scales");
  MOE_REQUIRE(T == 0 || x_t != MOE_E4M3 || x_scale, MOE_EINVAL, "E4M3 activations need tile scales");
  MOE_REQUIRE(ws && ws_bytes >= gemm_combine_workspace_bytes(T, K, Nr, Ns, d, I, tile_m, x_t, w_t), MOE_EWORKSPACE,
              "workspace smaller than moe_gemm_combine_workspace_bytes");
  const size_t P = permute_rows(T, K, Nr, Ns, tile_m);
  MOE_REQUIRE(P < (1ull << 31), MOE_EINVAL, "too many rows");
  const int tiles_max = (int)permute_tiles_max(T, K, Nr, Ns, tile_m);
  MOE_REQUIRE(tiles_max <= ffn_schedule_max_tiles(), MOE_EUNSUPPORTED,
              "more GEMM tiles than the work schedule holds");
  if (p == Path::BF16)
    MOE_REQUIRE(ffn_bf16_persistent_ok(d, I) && (unsigned long long)T * d * 2 < (1ull << 31) &&
                    (unsigned long long)P * I * 2 < (1ull << 31) && (unsigned long long)3 * I * d * 2 < (1ull << 31),
                MOE_EUNSUPPORTED, "bf16 fused combine needs d % 256 == 0, I % 128 == 0 and operands below 2 GiB");
  else
    MOE_REQUIRE(ffn_fp8_persistent_ok(d, I) && (unsigned long long)T * d < (1ull << 31) &&
                    (unsigned long long)P * I < (1ull << 31) && (unsigned long long)3 * I * d < (1ull << 31),
                MOE_EUNSUPPORTED, "fp8 fused combine needs d % 256 == 0, I % 256 == 0, d, I <= 8192");
  if (T == 0) return MOE_OK;
  hipStream_t st = as_stream(stream);
  int* ws_sched = static_cast<int*>(ws);
  uint8_t* ws_h = static_cast<uint8_t*>(ws) + gemm_sched_bytes(T, K, Nr, Ns, d, I, tile_m);
  const size_t g = gemm_workspace_bytes(T, K, Nr, Ns, d, I, tile_m, x_t, w_t);
  float* row_gate = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + (g + 255) / 256 * 256);
  launch_fused_combine_prep(u, u_t, inv_row, topk_gate, seg_offset, T, d, K, Nr, Ns, flags, out, row_gate, st);
  if (p == Path::BF16) {
    launch_ffn_bf16_persistent(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w13),
                               static_cast<const uint16_t*>(w2), row_token, tile_map, n_tiles, T, (long long)P, d, I,
                               Nr, tiles_max, reinterpret_cast<uint16_t*>(ws_h), nullptr, out, true, ws_sched, st,
                               row_gate);
  } else {
    uint8_t* h_codes = ws_h;
    float* h_scale = reinterpret_cast<float*>(ws_h + P * (size_t)I);
    launch_ffn_fp8_persistent(static_cast<const uint8_t*>(x), x_scale, static_cast<const uint8_t*>(w13), w13_scale,
                              static_cast<const uint8_t*>(w2), w2_scale, row_token, tile_map, n_tiles, T,
                              (long long)P, d, I, Nr, tiles_max, h_codes, h_scale, out, true, ws_sched, st, nullptr,
                              nullptr, row_gate);
  }
  return launch_status("moe_expert_gemm_combine");
}

}  // namespace moe
