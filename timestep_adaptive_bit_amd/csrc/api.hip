// extern "C" entry points of libtabit (declared in include/tabit.h).
//
// Every entry point validates its arguments completely before the first HIP
// call, records a message on the context for any failure, and enqueues its
// kernels on the caller's stream.  No device memory is allocated here.
#include "../../include/tabit.h"

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>

#include "tabit_internal.h"

namespace {

constexpr int kMaxK = 32768;
// Buffer descriptors address operands with 32-bit byte offsets; the top bit marks
// out-of-range reads, so every operand stays below 2^31 bytes.
constexpr size_t kMaxOperandBytes = 0x7FFFFFFFu;

int fail(tabit_ctx* ctx, int status, const char* fmt, ...) {
  if (ctx != nullptr) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    ctx->err = buf;
  }
  return status;
}

int hip_status(tabit_ctx* ctx, hipError_t e, const char* what) {
  if (e == hipSuccess) return TABIT_OK;
  return fail(ctx, TABIT_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_block(int b) { return b == 0 || b == 32 || b == 64 || b == 128; }

int check_k_shape(tabit_ctx* ctx, int M, int K, int had_block) {
  if (M < 0) return fail(ctx, TABIT_ESHAPE, "M must be >= 0 (got %d)", M);
  if (K < 32 || K > kMaxK || K % 32 != 0)
    return fail(ctx, TABIT_ESHAPE, "K must be a multiple of 32 in [32, %d] (got %d)", kMaxK, K);
  if (!valid_block(had_block))
    return fail(ctx, TABIT_ERANGE, "had_block must be 0, 32, 64 or 128 (got %d)", had_block);
  if (had_block > 0 && K % had_block != 0)
    return fail(ctx, TABIT_ESHAPE, "K (%d) must be a multiple of had_block (%d)", K, had_block);
  return TABIT_OK;
}

int check_gemm(tabit_ctx* ctx, const void* xq, const void* xs, const void* wq, const void* ws,
               int M, int N, int K, const void* y, const void* acc) {
  if (xq == nullptr || xs == nullptr || wq == nullptr || ws == nullptr)
    return fail(ctx, TABIT_EINVAL, "null input pointer");
  if (y == nullptr && acc == nullptr) return fail(ctx, TABIT_EINVAL, "no output requested");
  if (M < 0) return fail(ctx, TABIT_ESHAPE, "M must be >= 0 (got %d)", M);
  if (N < 0 || N % 32 != 0)
    return fail(ctx, TABIT_ESHAPE, "N must be a non-negative multiple of 32 (got %d)", N);
  if (K < 32 || K > kMaxK || K % 32 != 0)
    return fail(ctx, TABIT_ESHAPE, "K must be a multiple of 32 in [32, %d] (got %d)", kMaxK, K);
  if ((size_t)M * (size_t)K > kMaxOperandBytes || (size_t)N * (size_t)K > kMaxOperandBytes)
    return fail(ctx, TABIT_ESHAPE, "operands must stay below 2 GiB (M*K = %zu, N*K = %zu)",
                (size_t)M * (size_t)K, (size_t)N * (size_t)K);
  if (!aligned(xq, 16) || !aligned(wq, 16) || (y && !aligned(y, 16)) || (acc && !aligned(acc, 16)))
    return fail(ctx, TABIT_EALIGN, "matrices must be 16-byte aligned");
  return TABIT_OK;
}

// The GEMM of one INT8 layer-step on `path`: masked (w = int8 codes), bit-plane
// (same codes) or plane-major (w = the words of tabit_pack_weight_planes).  The
// tile configuration is the forced one, else the autotuned one, else the
// cost model's choice.
hipError_t launch_int8_family(const tabit_ctx* ctx, int path, const int8_t* xq, const float* sa,
                              const void* w, const float* sw, int M, int N, int K, int k,
                              uint16_t* y, int32_t* acc, hipStream_t s, int num_cus,
                              hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr,
                              const uint8_t* gate = nullptr) {
  if (path == TABIT_PATH_PLANES) {
    int cfg = ctx->force_plane_cfg;
    if (cfg < 0) cfg = ctx->tuned_cfg(TABIT_PATH_PLANES, M, N, K);
    if (cfg < 0) cfg = tabit::plane_config_choose(M, N, K, num_cus);
    return tabit::launch_gemm_planes(cfg, xq, sa, static_cast<const uint32_t*>(w), sw, M, N, K, k,
                                     y, acc, s, e0, e1, gate);
  }
  const bool bitserial = path == TABIT_PATH_BITSERIAL;
  int cfg = ctx->force_gemm_cfg;
  if (cfg < 0) cfg = ctx->tuned_cfg(bitserial ? 1 : 0, M, N, K);
  if (cfg < 0) cfg = tabit::gemm_config_choose(M, N, K, num_cus);
  return tabit::launch_gemm_i8(cfg, bitserial, xq, sa, static_cast<const int8_t*>(w), sw, M, N, K,
                               k, y, acc, s, e0, e1, gate);
}

bool valid_int8_path(int path) {
  return path == TABIT_PATH_MASKED || path == TABIT_PATH_BITSERIAL || path == TABIT_PATH_PLANES ||
         path == TABIT_PATH_HQDM;
}

int hqdm_cfg(const tabit_ctx* ctx, int M, int N, int K, int num_cus) {
  int cfg = ctx->force_hqdm_cfg;
  if (cfg < 0) cfg = tabit::hqdm_config_choose(M, N, K, num_cus);
  return cfg;
}

int gemm_i8_common(tabit_ctx* ctx, int path, const int8_t* x_q, const float* x_scale,
                   const void* w, const float* w_scale, int M, int N, int K, int k_bits,
                   uint16_t* y, int32_t* acc, void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  int st = check_gemm(ctx, x_q, x_scale, w, w_scale, M, N, K, y, acc);
  if (st != TABIT_OK) return st;
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4))
    return fail(ctx, TABIT_EALIGN, "scales must be 4-byte aligned");
  if (k_bits < 0 || k_bits > 7) return fail(ctx, TABIT_ERANGE, "k_bits must be in [0, 7] (got %d)", k_bits);
  if (M == 0 || N == 0) return TABIT_OK;
  static const char* const what[] = {"masked_qgemm launch", "qgemm_bitserial launch", "",
                                     "plane_qgemm launch"};
  return hip_status(ctx,
                    launch_int8_family(ctx, path, x_q, x_scale, w, w_scale, M, N, K, k_bits, y, acc,
                                       static_cast<hipStream_t>(stream), tabit::device_num_cus()),
                    what[path]);
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Bytes the compact workspace layout of one scheduled linear needs: the codes,
// then the scales (INT8; two code planes first on the HQ-DM path), or the FP4
// codes, then the E8M0 bytes (MXFP4), each section 256-byte aligned.
size_t compact_ws_bytes(int path, int fmt, int M, int K) {
  const size_t mk = (size_t)M * (size_t)K;
  if (fmt == TABIT_FMT_MXFP4) return align256(mk / 2) + align256(mk / 32);
  return (path == TABIT_PATH_HQDM ? 2 : 1) * align256(mk) + align256((size_t)M * 4);
}

// Every argument of one scheduled linear (step, layer) whose table entry is
// `fmt`, checked before anything is enqueued: shapes, alignment, operand
// sizes, and the weights the format needs.
int check_linear(tabit_ctx* ctx, int step, int layer, int path, int fmt, const uint16_t* x_bf16,
                 int M, int N, int K, int had_block, const int8_t* w_q, const float* w_scale,
                 const uint8_t* w_fp4, const uint8_t* w_e8m0, const uint16_t* y_bf16) {
  if (x_bf16 == nullptr || y_bf16 == nullptr) return fail(ctx, TABIT_EINVAL, "null pointer");
  int st = check_k_shape(ctx, M, K, had_block);
  if (st != TABIT_OK) return st;
  if (N < 0 || N % 32 != 0)
    return fail(ctx, TABIT_ESHAPE, "N must be a non-negative multiple of 32 (got %d)", N);
  if ((size_t)M * (size_t)K > kMaxOperandBytes || (size_t)N * (size_t)K > kMaxOperandBytes)
    return fail(ctx, TABIT_ESHAPE, "operands must stay below 2 GiB (M*K = %zu, N*K = %zu)",
                (size_t)M * (size_t)K, (size_t)N * (size_t)K);
  if (!aligned(x_bf16, 16) || !aligned(y_bf16, 16))
    return fail(ctx, TABIT_EALIGN, "x_bf16 and y_bf16 must be 16-byte aligned");
  if (fmt == TABIT_FMT_INT8) {
    if (w_q == nullptr || w_scale == nullptr)
      return fail(ctx, TABIT_EINVAL, "step %d layer %d is INT8 but w_q/w_scale are null", step, layer);
    if (!aligned(w_q, 16)) return fail(ctx, TABIT_EALIGN, "w_q must be 16-byte aligned");
    if (!aligned(w_scale, 4)) return fail(ctx, TABIT_EALIGN, "w_scale must be 4-byte aligned");
    if (path == TABIT_PATH_PLANES && N > 0 && tabit::planes_bytes(N, K) > kMaxOperandBytes)
      return fail(ctx, TABIT_ESHAPE, "the plane-major copy (%zu bytes) exceeds 2 GiB",
                  tabit::planes_bytes(N, K));
  } else {
    if (w_fp4 == nullptr || w_e8m0 == nullptr)
      return fail(ctx, TABIT_EINVAL, "step %d layer %d is MXFP4 but w_fp4/w_e8m0 are null", step, layer);
    if (had_block != 0 && had_block != 32)
      return fail(ctx, TABIT_ERANGE, "MXFP4 takes had_block 0 or 32 (got %d)", had_block);
    if (!aligned(w_fp4, 16)) return fail(ctx, TABIT_EALIGN, "w_fp4 must be 16-byte aligned");
  }
  return TABIT_OK;
}

// Enqueue one validated scheduled linear: quantize x into the workspace `ws`
// (layout of tabit_act_workspace_bytes), then the GEMM of the format and path.
int enqueue_linear(tabit_ctx* ctx, int path, int fmt, int k, const uint16_t* x_bf16, int M, int N,
                   int K, int had_block, const int8_t* w_q, const float* w_scale,
                   const uint8_t* w_fp4, const uint8_t* w_e8m0, uint8_t* ws, uint16_t* y_bf16,
                   void* stream, bool compact = false) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int num_cus = tabit::device_num_cus();
  const size_t mk = (size_t)M * (size_t)K;
  hipError_t e;
  if (fmt == TABIT_FMT_INT8) {
    int8_t* xq = reinterpret_cast<int8_t*>(ws);
    // scales after the HQ-DM path's second plane, or (compact) right after the codes
    const size_t sa_off = (compact && path != TABIT_PATH_HQDM ? 1 : 2) * align256(mk);
    float* sa = reinterpret_cast<float*>(ws + sa_off);
    if (path == TABIT_PATH_HQDM) {
      int8_t* xl = reinterpret_cast<int8_t*>(ws + align256(mk));
      e = tabit::launch_quant_hqdm(x_bf16, M, K, had_block, xq, xl, sa, s);
      if (e != hipSuccess) return hip_status(ctx, e, "HQ-DM quantizer launch");
      return hip_status(ctx,
                        tabit::launch_gemm_hqdm(hqdm_cfg(ctx, M, N, K, num_cus), xq, xl, sa, w_q,
                                                w_scale, M, N, K, k, y_bf16, nullptr, s),
                        "HQ-DM GEMM launch");
    }
    e = tabit::launch_quant_int8(x_bf16, M, K, had_block, 1.0f, xq, sa, s);
    if (e != hipSuccess) return hip_status(ctx, e, "quantizer launch");
    return hip_status(ctx,
                      launch_int8_family(ctx, path, xq, sa, w_q, w_scale, M, N, K, k, y_bf16,
                                         nullptr, s, num_cus),
                      "GEMM launch");
  }
  uint8_t* xf = ws;
  uint8_t* xe = ws + align256(mk / 2);
  e = tabit::launch_quant_mx(x_bf16, M, K, had_block, xf, xe, s);
  if (e != hipSuccess) return hip_status(ctx, e, "MX quantizer launch");
  int cfg = ctx->force_mx_cfg;
  if (cfg < 0) cfg = ctx->tuned_cfg(2, M, N, K);
  if (cfg < 0) cfg = tabit::mx_config_choose(M, N, K, num_cus);
  return hip_status(ctx,
                    tabit::launch_gemm_mxfp4(cfg, xf, xe, w_fp4, w_e8m0, M, N, K,
                                             1.0f / (float)(had_block > 0 ? had_block : 1), y_bf16,
                                             nullptr, s),
                    "MXFP4 GEMM launch");
}

}  // namespace

namespace tabit {

int device_num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace tabit

extern "C" {

int tabit_create(tabit_ctx** out) {
  if (out == nullptr) return TABIT_EINVAL;
  tabit_ctx* c = new (std::nothrow) tabit_ctx();
  if (c == nullptr) return TABIT_ENOMEM;
  *out = c;
  return TABIT_OK;
}

void tabit_destroy(tabit_ctx* ctx) { delete ctx; }

const char* tabit_last_error(const tabit_ctx* ctx) {
  if (ctx == nullptr) return "null tabit_ctx";
  return ctx->err.c_str();
}

const char* tabit_version(void) { return "tabit 0.1.0 gfx950"; }

int tabit_quantize_weights(tabit_ctx* ctx, const uint16_t* w_bf16, int N, int K, int had_block,
                           int8_t* w_q, float* w_scale, uint8_t* w_fp4, uint8_t* w_e8m0,
                           void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (w_bf16 == nullptr) return fail(ctx, TABIT_EINVAL, "null weight pointer");
  const bool want_i8 = w_q != nullptr || w_scale != nullptr;
  const bool want_mx = w_fp4 != nullptr || w_e8m0 != nullptr;
  if (want_i8 && (w_q == nullptr || w_scale == nullptr))
    return fail(ctx, TABIT_EINVAL, "w_q and w_scale must be given together");
  if (want_mx && (w_fp4 == nullptr || w_e8m0 == nullptr))
    return fail(ctx, TABIT_EINVAL, "w_fp4 and w_e8m0 must be given together");
  if (!want_i8 && !want_mx) return fail(ctx, TABIT_EINVAL, "no output requested");
  int st = check_k_shape(ctx, N, K, had_block);
  if (st != TABIT_OK) return st;
  if (want_mx && had_block != 0 && had_block != 32)
    return fail(ctx, TABIT_ERANGE, "the MXFP4 copy takes had_block 0 or 32 (got %d)", had_block);
  if (!aligned(w_bf16, 16) || (w_q && !aligned(w_q, 16)) || (w_fp4 && !aligned(w_fp4, 16)) ||
      (w_scale && !aligned(w_scale, 4)))
    return fail(ctx, TABIT_EALIGN, "misaligned pointer");
  if (N == 0) return TABIT_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (want_i8) {
    const float div = (float)(had_block > 0 ? had_block : 1);
    st = hip_status(ctx, tabit::launch_quant_int8(w_bf16, N, K, had_block, div, w_q, w_scale, s),
                    "quantize_weights launch");
    if (st != TABIT_OK) return st;
  }
  if (want_mx)
    return hip_status(ctx, tabit::launch_quant_mx(w_bf16, N, K, had_block, w_fp4, w_e8m0, s),
                      "quantize_weights (mxfp4) launch");
  return TABIT_OK;
}

int tabit_set_step_schedule(tabit_ctx* ctx, int num_steps, int num_layers, const uint8_t* k_bits,
                            const uint8_t* fmt) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (k_bits == nullptr) return fail(ctx, TABIT_EINVAL, "null k_bits table");
  if (num_steps < 1 || num_layers < 1)
    return fail(ctx, TABIT_ESHAPE, "schedule must be at least 1 x 1 (got %d x %d)", num_steps, num_layers);
  const size_t n = (size_t)num_steps * (size_t)num_layers;
  for (size_t i = 0; i < n; ++i) {
    if (k_bits[i] > 7) return fail(ctx, TABIT_ERANGE, "k_bits[%zu] = %d outside [0, 7]", i, k_bits[i]);
    if (fmt != nullptr && fmt[i] != TABIT_FMT_INT8 && fmt[i] != TABIT_FMT_MXFP4)
      return fail(ctx, TABIT_EINVAL, "fmt[%zu] = %d is not a known format", i, fmt[i]);
  }
  try {
    ctx->k_bits.assign(k_bits, k_bits + n);
    if (fmt != nullptr)
      ctx->fmt.assign(fmt, fmt + n);
    else
      ctx->fmt.assign(n, (uint8_t)TABIT_FMT_INT8);
  } catch (...) {
    ctx->k_bits.clear();
    ctx->fmt.clear();
    ctx->steps = ctx->layers = 0;
    return fail(ctx, TABIT_ENOMEM, "schedule allocation failed");
  }
  ctx->steps = num_steps;
  ctx->layers = num_layers;
  return TABIT_OK;
}

int tabit_schedule_lookup(const tabit_ctx* ctx, int step, int layer, int* k_bits, int* fmt) {
  if (ctx == nullptr || k_bits == nullptr || fmt == nullptr) return TABIT_EINVAL;
  tabit_ctx* c = const_cast<tabit_ctx*>(ctx);
  if (ctx->steps == 0) return fail(c, TABIT_ENOSCHED, "no schedule installed");
  if (step < 0 || step >= ctx->steps || layer < 0 || layer >= ctx->layers)
    return fail(c, TABIT_ENOSCHED, "(step %d, layer %d) outside the %d x %d schedule", step, layer,
                ctx->steps, ctx->layers);
  const size_t i = (size_t)step * ctx->layers + layer;
  *k_bits = ctx->k_bits[i];
  *fmt = ctx->fmt[i];
  return TABIT_OK;
}

int tabit_hadamard_quant_act(tabit_ctx* ctx, const uint16_t* x_bf16, int M, int K, int had_block,
                             int fmt, void* x_q, void* x_scale, void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (x_bf16 == nullptr || x_q == nullptr || x_scale == nullptr)
    return fail(ctx, TABIT_EINVAL, "null pointer");
  if (fmt != TABIT_FMT_INT8 && fmt != TABIT_FMT_MXFP4)
    return fail(ctx, TABIT_EINVAL, "unknown fmt %d", fmt);
  int st = check_k_shape(ctx, M, K, had_block);
  if (st != TABIT_OK) return st;
  if (fmt == TABIT_FMT_MXFP4 && had_block != 0 && had_block != 32)
    return fail(ctx, TABIT_ERANGE, "MXFP4 takes had_block 0 or 32 (got %d)", had_block);
  if (!aligned(x_bf16, 16) || !aligned(x_q, 16) || (fmt == TABIT_FMT_INT8 && !aligned(x_scale, 4)))
    return fail(ctx, TABIT_EALIGN, "misaligned pointer");
  if (M == 0) return TABIT_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fmt == TABIT_FMT_INT8)
    return hip_status(ctx,
                      tabit::launch_quant_int8(x_bf16, M, K, had_block, 1.0f,
                                               static_cast<int8_t*>(x_q),
                                               static_cast<float*>(x_scale), s),
                      "hadamard_quant_act launch");
  return hip_status(ctx,
                    tabit::launch_quant_mx(x_bf16, M, K, had_block, static_cast<uint8_t*>(x_q),
                                           static_cast<uint8_t*>(x_scale), s),
                    "hadamard_quant_act (mxfp4) launch");
}

int tabit_masked_qgemm(tabit_ctx* ctx, const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                       const float* w_scale, int M, int N, int K, int k_bits, uint16_t* y_bf16,
                       int32_t* acc, void* stream) {
  return gemm_i8_common(ctx, TABIT_PATH_MASKED, x_q, x_scale, w_q, w_scale, M, N, K, k_bits, y_bf16,
                        acc, stream);
}

int tabit_qgemm_bitserial(tabit_ctx* ctx, const int8_t* x_q, const float* x_scale,
                          const int8_t* w_q, const float* w_scale, int M, int N, int K, int k_bits,
                          uint16_t* y_bf16, int32_t* acc, void* stream) {
  return gemm_i8_common(ctx, TABIT_PATH_BITSERIAL, x_q, x_scale, w_q, w_scale, M, N, K, k_bits,
                        y_bf16, acc, stream);
}

int tabit_pack_weight_planes(tabit_ctx* ctx, const int8_t* w_q, int N, int K, uint32_t* w_planes,
                             void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (w_q == nullptr || w_planes == nullptr) return fail(ctx, TABIT_EINVAL, "null pointer");
  if (N < 0 || N % 32 != 0)
    return fail(ctx, TABIT_ESHAPE, "N must be a non-negative multiple of 32 (got %d)", N);
  if (K < 32 || K > kMaxK || K % 32 != 0)
    return fail(ctx, TABIT_ESHAPE, "K must be a multiple of 32 in [32, %d] (got %d)", kMaxK, K);
  if (tabit::planes_bytes(N, K) > kMaxOperandBytes)
    return fail(ctx, TABIT_ESHAPE, "the plane-major copy (%zu bytes) exceeds 2 GiB",
                tabit::planes_bytes(N, K));
  if (!aligned(w_q, 16) || !aligned(w_planes, 16))
    return fail(ctx, TABIT_EALIGN, "w_q and w_planes must be 16-byte aligned");
  if (N == 0) return TABIT_OK;
  return hip_status(ctx, tabit::launch_pack_planes(w_q, N, K, w_planes, static_cast<hipStream_t>(stream)),
                    "pack_weight_planes launch");
}

size_t tabit_weight_planes_bytes(int N, int K) {
  if (N <= 0 || K <= 0) return 0;
  return tabit::planes_bytes(N, K);
}

int tabit_plane_qgemm(tabit_ctx* ctx, const int8_t* x_q, const float* x_scale,
                      const uint32_t* w_planes, const float* w_scale, int M, int N, int K,
                      int k_bits, uint16_t* y_bf16, int32_t* acc, void* stream) {
  if (ctx != nullptr && N > 0 && K > 0 && tabit::planes_bytes(N, K) > kMaxOperandBytes)
    return fail(ctx, TABIT_ESHAPE, "the plane-major copy (%zu bytes) exceeds 2 GiB",
                tabit::planes_bytes(N, K));
  return gemm_i8_common(ctx, TABIT_PATH_PLANES, x_q, x_scale, w_planes, w_scale, M, N, K, k_bits,
                        y_bf16, acc, stream);
}

int tabit_mxfp4_qgemm(tabit_ctx* ctx, const uint8_t* x_fp4, const uint8_t* x_e8m0,
                      const uint8_t* w_fp4, const uint8_t* w_e8m0, int M, int N, int K,
                      float out_scale, uint16_t* y_bf16, float* acc_f32, void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  int st = check_gemm(ctx, x_fp4, x_e8m0, w_fp4, w_e8m0, M, N, K, y_bf16, acc_f32);
  if (st != TABIT_OK) return st;
  if (!(out_scale == out_scale)) return fail(ctx, TABIT_EINVAL, "out_scale is NaN");
  if (M == 0 || N == 0) return TABIT_OK;
  int cfg = ctx->force_mx_cfg;
  if (cfg < 0) cfg = ctx->tuned_cfg(2, M, N, K);
  if (cfg < 0) cfg = tabit::mx_config_choose(M, N, K, tabit::device_num_cus());
  return hip_status(ctx,
                    tabit::launch_gemm_mxfp4(cfg, x_fp4, x_e8m0, w_fp4, w_e8m0, M, N, K, out_scale,
                                             y_bf16, acc_f32, static_cast<hipStream_t>(stream)),
                    "mxfp4_qgemm launch");
}

int tabit_gelu_quant_act(tabit_ctx* ctx, const uint16_t* x_bf16, int M, int K, int had_block,
                         int fmt, void* x_q, void* x_scale, void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (x_bf16 == nullptr || x_q == nullptr || x_scale == nullptr)
    return fail(ctx, TABIT_EINVAL, "null pointer");
  if (fmt != TABIT_FMT_INT8 && fmt != TABIT_FMT_MXFP4)
    return fail(ctx, TABIT_EINVAL, "unknown fmt %d", fmt);
  int st = check_k_shape(ctx, M, K, had_block);
  if (st != TABIT_OK) return st;
  if (fmt == TABIT_FMT_MXFP4 && had_block != 0 && had_block != 32)
    return fail(ctx, TABIT_ERANGE, "MXFP4 takes had_block 0 or 32 (got %d)", had_block);
  if ((size_t)M * (size_t)K > kMaxOperandBytes)
    return fail(ctx, TABIT_ESHAPE, "activations must stay below 2 GiB");
  if (!aligned(x_bf16, 16) || !aligned(x_q, 16) || (fmt == TABIT_FMT_INT8 && !aligned(x_scale, 4)))
    return fail(ctx, TABIT_EALIGN, "misaligned pointer");
  if (M == 0) return TABIT_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fmt == TABIT_FMT_INT8)
    return hip_status(ctx,
                      tabit::launch_quant_gelu_int8(x_bf16, M, K, had_block,
                                                    static_cast<int8_t*>(x_q),
                                                    static_cast<float*>(x_scale), s),
                      "gelu_quant_act launch");
  return hip_status(ctx,
                    tabit::launch_quant_gelu_mx(x_bf16, M, K, had_block, static_cast<uint8_t*>(x_q),
                                                static_cast<uint8_t*>(x_scale), s),
                    "gelu_quant_act (mxfp4) launch");
}

int tabit_hqdm_quant_act(tabit_ctx* ctx, const uint16_t* x_bf16, int M, int K, int had_block,
                         int8_t* x_hi, int8_t* x_lo, float* x_scale, void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (x_bf16 == nullptr || x_hi == nullptr || x_lo == nullptr || x_scale == nullptr)
    return fail(ctx, TABIT_EINVAL, "null pointer");
  int st = check_k_shape(ctx, M, K, had_block);
  if (st != TABIT_OK) return st;
  if ((size_t)M * (size_t)K > kMaxOperandBytes)
    return fail(ctx, TABIT_ESHAPE, "activations must stay below 2 GiB");
  if (!aligned(x_bf16, 16) || !aligned(x_hi, 16) || !aligned(x_lo, 16) || !aligned(x_scale, 4))
    return fail(ctx, TABIT_EALIGN, "misaligned pointer");
  if (M == 0) return TABIT_OK;
  return hip_status(ctx,
                    tabit::launch_quant_hqdm(x_bf16, M, K, had_block, x_hi, x_lo, x_scale,
                                             static_cast<hipStream_t>(stream)),
                    "hqdm_quant_act launch");
}

int tabit_hqdm_qgemm(tabit_ctx* ctx, const int8_t* x_hi, const int8_t* x_lo, const float* x_scale,
                     const int8_t* w_q, const float* w_scale, int M, int N, int K, int k_bits,
                     uint16_t* y_bf16, int64_t* acc, void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (x_lo == nullptr) return fail(ctx, TABIT_EINVAL, "null input pointer");
  int st = check_gemm(ctx, x_hi, x_scale, w_q, w_scale, M, N, K, y_bf16, acc);
  if (st != TABIT_OK) return st;
  if (!aligned(x_lo, 16)) return fail(ctx, TABIT_EALIGN, "matrices must be 16-byte aligned");
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4))
    return fail(ctx, TABIT_EALIGN, "scales must be 4-byte aligned");
  if (k_bits < 0 || k_bits > 7) return fail(ctx, TABIT_ERANGE, "k_bits must be in [0, 7] (got %d)", k_bits);
  if (M == 0 || N == 0) return TABIT_OK;
  const int num_cus = tabit::device_num_cus();
  return hip_status(ctx,
                    tabit::launch_gemm_hqdm(hqdm_cfg(ctx, M, N, K, num_cus), x_hi, x_lo, x_scale,
                                            w_q, w_scale, M, N, K, k_bits, y_bf16,
                                            reinterpret_cast<long long*>(acc),
                                            static_cast<hipStream_t>(stream)),
                    "hqdm_qgemm launch");
}

int tabit_hqdm_config_info(int index, int* bm, int* bn) {
  if (index < 0) return tabit::hqdm_config_count();
  if (index >= tabit::hqdm_config_count() || bm == nullptr || bn == nullptr) return TABIT_EINVAL;
  const tabit::GemmConfig c = tabit::hqdm_config(index);
  *bm = c.bm;
  *bn = c.bn;
  return TABIT_OK;
}

size_t tabit_act_workspace_bytes(int M, int K) {
  if (M <= 0 || K <= 0) return 0;
  const size_t mk = (size_t)M * (size_t)K;
  const size_t i8 = 2 * align256(mk) + align256((size_t)M * 4);   // HQ-DM: two planes
  const size_t mx = align256(mk / 2) + align256(mk / 32);
  return i8 > mx ? i8 : mx;
}

int tabit_scheduled_linear(tabit_ctx* ctx, int step, int layer, int path, const uint16_t* x_bf16,
                           int M, int N, int K, int had_block, const int8_t* w_q,
                           const float* w_scale, const uint8_t* w_fp4, const uint8_t* w_e8m0,
                           void* act_ws, size_t act_ws_bytes, uint16_t* y_bf16, void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (!valid_int8_path(path)) return fail(ctx, TABIT_EINVAL, "unknown path %d", path);
  int k = 0, fmt = 0;
  int st = tabit_schedule_lookup(ctx, step, layer, &k, &fmt);
  if (st != TABIT_OK) return st;
  if (act_ws == nullptr) return fail(ctx, TABIT_EINVAL, "null pointer");
  if (!aligned(act_ws, 16)) return fail(ctx, TABIT_EALIGN, "act_ws must be 16-byte aligned");
  if (act_ws_bytes < tabit_act_workspace_bytes(M, K))
    return fail(ctx, TABIT_ESHAPE, "act_ws holds %zu bytes, %zu needed", act_ws_bytes,
                tabit_act_workspace_bytes(M, K));
  st = check_linear(ctx, step, layer, path, fmt, x_bf16, M, N, K, had_block, w_q, w_scale, w_fp4,
                    w_e8m0, y_bf16);
  if (st != TABIT_OK) return st;
  if (M == 0 || N == 0) return TABIT_OK;
  return enqueue_linear(ctx, path, fmt, k, x_bf16, M, N, K, had_block, w_q, w_scale, w_fp4, w_e8m0,
                        static_cast<uint8_t*>(act_ws), y_bf16, stream);
}

// Device scratch of tabit_scheduled_linear_noalloc: a file-scope array, so the
// entry point never allocates.  Each GPU the library runs on holds its own copy
// (loaded with the code object, kept until the process ends); host code reaches
// it only through the address hipGetSymbolAddress returns on that device.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// The current device's address of `scratch`, looked up once per device with
// that device current.
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

size_t tabit_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int tabit_scheduled_linear_noalloc(tabit_ctx* ctx, int step, int layer, int path,
                                   const uint16_t* x_bf16, int M, int N, int K, int had_block,
                                   const int8_t* w_q, const float* w_scale, const uint8_t* w_fp4,
                                   const uint8_t* w_e8m0, uint16_t* y_bf16, void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (!valid_int8_path(path)) return fail(ctx, TABIT_EINVAL, "unknown path %d", path);
  int k = 0, fmt = 0;
  int st = tabit_schedule_lookup(ctx, step, layer, &k, &fmt);
  if (st != TABIT_OK) return st;
  st = check_linear(ctx, step, layer, path, fmt, x_bf16, M, N, K, had_block, w_q, w_scale, w_fp4,
                    w_e8m0, y_bf16);
  if (st != TABIT_OK) return st;
  const size_t need = compact_ws_bytes(path, fmt, M, K);
  if (need > kNoAllocScratchBytes)
    return fail(ctx, TABIT_ESHAPE,
                "%d x %d activations need %zu bytes of scratch; the static scratch holds %zu",
                M, K, need, kNoAllocScratchBytes);
  if (M == 0 || N == 0) return TABIT_OK;
  void* ws = nullptr;
  st = hip_status(ctx, scratch_on_current_device(&ws), "scratch address lookup");
  if (st != TABIT_OK) return st;
  return enqueue_linear(ctx, path, fmt, k, x_bf16, M, N, K, had_block, w_q, w_scale, w_fp4, w_e8m0,
                        static_cast<uint8_t*>(ws), y_bf16, stream, /*compact=*/true);
}

size_t tabit_dmpq_workspace_bytes(int M) { return tabit::dmpq_workspace_bytes(M); }

int tabit_dmpq_select(tabit_ctx* ctx, const uint16_t* x_in, const uint16_t* x_out, int M, int H,
                      const float* theta, int n_layers, uint8_t* fmt, double* gamma, void* ws,
                      size_t ws_bytes, void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (x_in == nullptr || x_out == nullptr || ws == nullptr) return fail(ctx, TABIT_EINVAL, "null pointer");
  if (n_layers < 0) return fail(ctx, TABIT_EINVAL, "n_layers must be >= 0 (got %d)", n_layers);
  if (n_layers > 0 && (theta == nullptr || fmt == nullptr))
    return fail(ctx, TABIT_EINVAL, "theta and fmt are required when n_layers > 0");
  if (n_layers == 0 && gamma == nullptr) return fail(ctx, TABIT_EINVAL, "no output requested");
  if (M < 1) return fail(ctx, TABIT_ESHAPE, "M must be >= 1 (got %d)", M);
  if (H < 16 || H > kMaxK || H % 16 != 0)
    return fail(ctx, TABIT_ESHAPE, "H must be a multiple of 16 in [16, %d] (got %d)", kMaxK, H);
  if ((size_t)M * (size_t)H * 2 > kMaxOperandBytes)
    return fail(ctx, TABIT_ESHAPE, "hidden states must stay below 2 GiB");
  if (!aligned(x_in, 16) || !aligned(x_out, 16) || !aligned(ws, 16) ||
      (theta && !aligned(theta, 4)) || (gamma && !aligned(gamma, 8)))
    return fail(ctx, TABIT_EALIGN, "misaligned pointer");
  if (ws_bytes < tabit::dmpq_workspace_bytes(M))
    return fail(ctx, TABIT_ESHAPE, "ws holds %zu bytes, %zu needed", ws_bytes,
                tabit::dmpq_workspace_bytes(M));
  return hip_status(ctx,
                    tabit::launch_dmpq_select(x_in, x_out, M, H, static_cast<double*>(ws), theta,
                                              n_layers, fmt, gamma, static_cast<hipStream_t>(stream)),
                    "dmpq_select launch");
}

int tabit_gated_linear(tabit_ctx* ctx, const uint8_t* fmt_dev, int k_bits, int path,
                       const uint16_t* x_bf16, int M, int N, int K, int had_block,
                       const void* w_q, const float* w_scale, const uint8_t* w_fp4,
                       const uint8_t* w_e8m0, void* act_ws, size_t act_ws_bytes, uint16_t* y_bf16,
                       void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (fmt_dev == nullptr || x_bf16 == nullptr || y_bf16 == nullptr || act_ws == nullptr ||
      w_q == nullptr || w_scale == nullptr || w_fp4 == nullptr || w_e8m0 == nullptr)
    return fail(ctx, TABIT_EINVAL, "null pointer (both weight formats are required)");
  if (path != TABIT_PATH_MASKED && path != TABIT_PATH_PLANES)
    return fail(ctx, TABIT_EINVAL, "gated linear takes the masked or plane-major path (got %d)", path);
  if (k_bits < 0 || k_bits > 7) return fail(ctx, TABIT_ERANGE, "k_bits must be in [0, 7] (got %d)", k_bits);
  int st = check_k_shape(ctx, M, K, had_block);
  if (st != TABIT_OK) return st;
  if (had_block != 0 && had_block != 32)
    return fail(ctx, TABIT_ERANGE, "MXFP4 takes had_block 0 or 32 (got %d)", had_block);
  if (N < 0 || N % 32 != 0)
    return fail(ctx, TABIT_ESHAPE, "N must be a non-negative multiple of 32 (got %d)", N);
  if ((size_t)M * (size_t)K > kMaxOperandBytes || (size_t)N * (size_t)K > kMaxOperandBytes ||
      (path == TABIT_PATH_PLANES && N > 0 && tabit::planes_bytes(N, K) > kMaxOperandBytes))
    return fail(ctx, TABIT_ESHAPE, "operands must stay below 2 GiB");
  if (!aligned(x_bf16, 16) || !aligned(y_bf16, 16) || !aligned(act_ws, 16) || !aligned(w_q, 16) ||
      !aligned(w_fp4, 16) || !aligned(w_scale, 4))
    return fail(ctx, TABIT_EALIGN, "misaligned pointer");
  if (act_ws_bytes < tabit_act_workspace_bytes(M, K))
    return fail(ctx, TABIT_ESHAPE, "act_ws holds %zu bytes, %zu needed", act_ws_bytes,
                tabit_act_workspace_bytes(M, K));
  if (M == 0 || N == 0) return TABIT_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(act_ws);
  const size_t mk = (size_t)M * (size_t)K;
  const int num_cus = tabit::device_num_cus();
  // INT8 branch: runs when *fmt_dev == TABIT_FMT_INT8
  int8_t* xq = reinterpret_cast<int8_t*>(ws);
  float* sa = reinterpret_cast<float*>(ws + 2 * align256(mk));
  hipError_t e = tabit::launch_quant_int8(x_bf16, M, K, had_block, 1.0f, xq, sa, s, fmt_dev);
  if (e != hipSuccess) return hip_status(ctx, e, "gated quantizer launch");
  e = launch_int8_family(ctx, path, xq, sa, w_q, w_scale, M, N, K, k_bits, y_bf16, nullptr, s,
                         num_cus, nullptr, nullptr, fmt_dev);
  if (e != hipSuccess) return hip_status(ctx, e, "gated GEMM launch");
  // MXFP4 branch: runs when *fmt_dev == TABIT_FMT_MXFP4 (same workspace; only one branch runs)
  uint8_t* xf = ws;
  uint8_t* xe = ws + align256(mk / 2);
  e = tabit::launch_quant_mx(x_bf16, M, K, had_block, xf, xe, s, fmt_dev);
  if (e != hipSuccess) return hip_status(ctx, e, "gated MX quantizer launch");
  int cfg = ctx->force_mx_cfg;
  if (cfg < 0) cfg = ctx->tuned_cfg(2, M, N, K);
  if (cfg < 0) cfg = tabit::mx_config_choose(M, N, K, num_cus);
  e = tabit::launch_gemm_mxfp4(cfg, xf, xe, w_fp4, w_e8m0, M, N, K,
                               1.0f / (float)(had_block > 0 ? had_block : 1), y_bf16, nullptr, s,
                               nullptr, nullptr, fmt_dev);
  return hip_status(ctx, e, "gated MXFP4 GEMM launch");
}

int tabit_run_schedule(tabit_ctx* ctx, int first_step, int num_steps, const tabit_layer* layers,
                       int num_layers, const uint16_t* const* x_bf16, int had_block, int path,
                       void* act_ws, size_t act_ws_bytes, void* const* gemm_events, void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (layers == nullptr || x_bf16 == nullptr || act_ws == nullptr)
    return fail(ctx, TABIT_EINVAL, "null pointer");
  if (!valid_int8_path(path)) return fail(ctx, TABIT_EINVAL, "unknown path %d", path);
  if (ctx->steps == 0) return fail(ctx, TABIT_ENOSCHED, "no schedule installed");
  if (num_layers != ctx->layers)
    return fail(ctx, TABIT_ESHAPE, "%d layers given, schedule has %d", num_layers, ctx->layers);
  if (num_steps < 0 || first_step < 0 || first_step + num_steps > ctx->steps)
    return fail(ctx, TABIT_ENOSCHED, "steps [%d, %d) outside the %d-step schedule", first_step,
                first_step + num_steps, ctx->steps);
  if (!aligned(act_ws, 16)) return fail(ctx, TABIT_EALIGN, "act_ws must be 16-byte aligned");
  if (!valid_block(had_block))
    return fail(ctx, TABIT_ERANGE, "had_block must be 0, 32, 64 or 128 (got %d)", had_block);
  // validate everything before the first launch
  for (int l = 0; l < num_layers; ++l) {
    const tabit_layer& L = layers[l];
    int st = check_k_shape(ctx, L.M, L.K, had_block);
    if (st != TABIT_OK) return st;
    if (L.input_from < 0 || L.input_from > l)
      return fail(ctx, TABIT_EINVAL, "layer %d: input_from %d must name an earlier layer (1..%d) or 0",
                  l, L.input_from, l);
    if (L.input_act != TABIT_ACT_NONE && L.input_act != TABIT_ACT_GELU)
      return fail(ctx, TABIT_EINVAL, "layer %d: unknown input_act %d", l, L.input_act);
    if (L.input_from > 0) {
      const tabit_layer& P = layers[L.input_from - 1];
      if (P.M != L.M || P.N != L.K)
        return fail(ctx, TABIT_ESHAPE, "layer %d: input from layer %d is %d x %d, needs %d x %d", l,
                    L.input_from - 1, P.M, P.N, L.M, L.K);
    }
    if (L.input_act == TABIT_ACT_GELU && path == TABIT_PATH_HQDM)
      return fail(ctx, TABIT_EINVAL, "layer %d: the HQ-DM path has no GELU-fused quantizer", l);
    if (L.N < 0 || L.N % 32 != 0)
      return fail(ctx, TABIT_ESHAPE, "layer %d: N must be a non-negative multiple of 32", l);
    if (L.y_bf16 == nullptr || !aligned(L.y_bf16, 16))
      return fail(ctx, TABIT_EINVAL, "layer %d: missing or misaligned output", l);
    if ((size_t)L.M * (size_t)L.K > kMaxOperandBytes || (size_t)L.N * (size_t)L.K > kMaxOperandBytes ||
        (path == TABIT_PATH_PLANES && L.N > 0 && tabit::planes_bytes(L.N, L.K) > kMaxOperandBytes))
      return fail(ctx, TABIT_ESHAPE, "layer %d: operands must stay below 2 GiB", l);
    if (act_ws_bytes < tabit_act_workspace_bytes(L.M, L.K))
      return fail(ctx, TABIT_ESHAPE, "layer %d: act_ws holds %zu bytes, %zu needed", l,
                  act_ws_bytes, tabit_act_workspace_bytes(L.M, L.K));
    for (int t = first_step; t < first_step + num_steps; ++t) {
      const size_t i = (size_t)t * ctx->layers + l;
      const uint16_t* x = L.input_from > 0 ? layers[L.input_from - 1].y_bf16
                                           : x_bf16[(size_t)(t - first_step) * num_layers + l];
      if (x == nullptr || !aligned(x, 16))
        return fail(ctx, TABIT_EINVAL, "step %d layer %d: missing or misaligned input", t, l);
      if (ctx->fmt[i] == TABIT_FMT_INT8) {
        if (L.w_q == nullptr || L.w_scale == nullptr || !aligned(L.w_q, 16))
          return fail(ctx, TABIT_EINVAL, "layer %d: INT8 step %d without INT8 weights", l, t);
      } else {
        if (L.w_fp4 == nullptr || L.w_e8m0 == nullptr || !aligned(L.w_fp4, 16))
          return fail(ctx, TABIT_EINVAL, "layer %d: MXFP4 step %d without the MX copy", l, t);
        if (had_block != 0 && had_block != 32)
          return fail(ctx, TABIT_ERANGE, "MXFP4 takes had_block 0 or 32 (got %d)", had_block);
      }
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(act_ws);
  const int num_cus = tabit::device_num_cus();
  for (int t = first_step; t < first_step + num_steps; ++t) {
    for (int l = 0; l < num_layers; ++l) {
      const tabit_layer& L = layers[l];
      const size_t li = (size_t)(t - first_step) * num_layers + l;
      const size_t i = (size_t)t * ctx->layers + l;
      const uint16_t* x = L.input_from > 0 ? layers[L.input_from - 1].y_bf16 : x_bf16[li];
      const bool gelu = L.input_act == TABIT_ACT_GELU;
      hipEvent_t e0 = gemm_events ? static_cast<hipEvent_t>(gemm_events[2 * li]) : nullptr;
      hipEvent_t e1 = gemm_events ? static_cast<hipEvent_t>(gemm_events[2 * li + 1]) : nullptr;
      if (L.M == 0 || L.N == 0) continue;
      const size_t mk = (size_t)L.M * (size_t)L.K;
      hipError_t e;
      if (ctx->fmt[i] == TABIT_FMT_INT8) {
        int8_t* xq = reinterpret_cast<int8_t*>(ws);
        float* sa = reinterpret_cast<float*>(ws + 2 * align256(mk));
        if (path == TABIT_PATH_HQDM) {
          int8_t* xl = reinterpret_cast<int8_t*>(ws + align256(mk));
          e = tabit::launch_quant_hqdm(x, L.M, L.K, had_block, xq, xl, sa, s);
          if (e != hipSuccess) return hip_status(ctx, e, "run_schedule HQ-DM quantizer launch");
          e = tabit::launch_gemm_hqdm(hqdm_cfg(ctx, L.M, L.N, L.K, num_cus), xq, xl, sa, L.w_q,
                                      L.w_scale, L.M, L.N, L.K, ctx->k_bits[i], L.y_bf16, nullptr,
                                      s, e0, e1);
        } else {
          e = gelu ? tabit::launch_quant_gelu_int8(x, L.M, L.K, had_block, xq, sa, s)
                   : tabit::launch_quant_int8(x, L.M, L.K, had_block, 1.0f, xq, sa, s);
          if (e != hipSuccess) return hip_status(ctx, e, "run_schedule quantizer launch");
          e = launch_int8_family(ctx, path, xq, sa, L.w_q, L.w_scale, L.M, L.N, L.K, ctx->k_bits[i],
                                 L.y_bf16, nullptr, s, num_cus, e0, e1);
        }
        if (e != hipSuccess) return hip_status(ctx, e, "run_schedule GEMM launch");
      } else {
        uint8_t* xf = ws;
        uint8_t* xe = ws + align256(mk / 2);
        e = gelu ? tabit::launch_quant_gelu_mx(x, L.M, L.K, had_block, xf, xe, s)
                 : tabit::launch_quant_mx(x, L.M, L.K, had_block, xf, xe, s);
        if (e != hipSuccess) return hip_status(ctx, e, "run_schedule MX quantizer launch");
        int cfg = ctx->force_mx_cfg;
        if (cfg < 0) cfg = ctx->tuned_cfg(2, L.M, L.N, L.K);
        if (cfg < 0) cfg = tabit::mx_config_choose(L.M, L.N, L.K, num_cus);
        e = tabit::launch_gemm_mxfp4(cfg, xf, xe, L.w_fp4, L.w_e8m0, L.M, L.N, L.K,
                                     1.0f / (float)(had_block > 0 ? had_block : 1), L.y_bf16,
                                     nullptr, s, e0, e1);
        if (e != hipSuccess) return hip_status(ctx, e, "run_schedule MXFP4 GEMM launch");
      }
    }
  }
  return TABIT_OK;
}

int tabit_autotune_gemm(tabit_ctx* ctx, int path, const void* x_q, const void* x_scale,
                        const void* w_q, const void* w_scale, int M, int N, int K, int k_bits,
                        uint16_t* y_bf16, int reps, int* best_cfg, void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (path < 0 || path > 3) return fail(ctx, TABIT_EINVAL, "unknown GEMM path %d", path);
  if (y_bf16 == nullptr) return fail(ctx, TABIT_EINVAL, "autotune needs y_bf16");
  if (reps < 1) return fail(ctx, TABIT_EINVAL, "reps must be >= 1");
  int st = check_gemm(ctx, x_q, x_scale, w_q, w_scale, M, N, K, y_bf16, nullptr);
  if (st != TABIT_OK) return st;
  if (k_bits < 0 || k_bits > 7) return fail(ctx, TABIT_ERANGE, "k_bits must be in [0, 7] (got %d)", k_bits);
  if (M == 0 || N == 0) return TABIT_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n = path == 2   ? tabit::mx_config_count()
                : path == 3 ? tabit::plane_config_count()
                            : tabit::gemm_config_count();
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return hip_status(ctx, e, "autotune event create");
  }
  auto launch = [&](int cfg) {
    if (path == 2)
      return tabit::launch_gemm_mxfp4(cfg, static_cast<const uint8_t*>(x_q),
                                      static_cast<const uint8_t*>(x_scale),
                                      static_cast<const uint8_t*>(w_q),
                                      static_cast<const uint8_t*>(w_scale), M, N, K, 1.0f, y_bf16,
                                      nullptr, s);
    if (path == 3)
      return tabit::launch_gemm_planes(cfg, static_cast<const int8_t*>(x_q),
                                       static_cast<const float*>(x_scale),
                                       static_cast<const uint32_t*>(w_q),
                                       static_cast<const float*>(w_scale), M, N, K, k_bits, y_bf16,
                                       nullptr, s);
    return tabit::launch_gemm_i8(cfg, path == 1, static_cast<const int8_t*>(x_q),
                                 static_cast<const float*>(x_scale), static_cast<const int8_t*>(w_q),
                                 static_cast<const float*>(w_scale), M, N, K, k_bits, y_bf16,
                                 nullptr, s);
  };
  int best = -1;
  float best_ms = 0.0f;
  for (int cfg = 0; cfg < n && e == hipSuccess; ++cfg) {
    e = launch(cfg);                                     // warm-up
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch(cfg);
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && (best < 0 || ms < best_ms)) {
      best = cfg;
      best_ms = ms;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return hip_status(ctx, e, "autotune");
  ctx->tuned[std::make_tuple(path, M, N, K)] = best;
  if (best_cfg) *best_cfg = best;
  return TABIT_OK;
}

int tabit_set_option(tabit_ctx* ctx, int option, int value) {
  if (ctx == nullptr) return TABIT_EINVAL;
  switch (option) {
    case TABIT_OPT_GEMM_CONFIG:
      if (value < -1 || value >= tabit::gemm_config_count())
        return fail(ctx, TABIT_EINVAL, "GEMM config %d out of range", value);
      ctx->force_gemm_cfg = value;
      return TABIT_OK;
    case TABIT_OPT_MXFP4_CONFIG:
      if (value < -1 || value >= tabit::mx_config_count())
        return fail(ctx, TABIT_EINVAL, "MXFP4 config %d out of range", value);
      ctx->force_mx_cfg = value;
      return TABIT_OK;
    case TABIT_OPT_PLANE_CONFIG:
      if (value < -1 || value >= tabit::plane_config_count())
        return fail(ctx, TABIT_EINVAL, "plane GEMM config %d out of range", value);
      ctx->force_plane_cfg = value;
      return TABIT_OK;
    case TABIT_OPT_HQDM_CONFIG:
      if (value < -1 || value >= tabit::hqdm_config_count())
        return fail(ctx, TABIT_EINVAL, "HQ-DM GEMM config %d out of range", value);
      ctx->force_hqdm_cfg = value;
      return TABIT_OK;
    default:
      return fail(ctx, TABIT_EINVAL, "unknown option %d", option);
  }
}

int tabit_gemm_config_info(int index, int* bm, int* bn, int* k_groups) {
  if (index < 0) return tabit::gemm_config_count();
  if (index >= tabit::gemm_config_count() || bm == nullptr || bn == nullptr || k_groups == nullptr)
    return TABIT_EINVAL;
  const tabit::GemmConfig c = tabit::gemm_config(index);
  *bm = c.bm;
  *bn = c.bn;
  *k_groups = c.k_groups;
  return TABIT_OK;
}

int tabit_mxfp4_config_info(int index, int* bm, int* bn) {
  if (index < 0) return tabit::mx_config_count();
  if (index >= tabit::mx_config_count() || bm == nullptr || bn == nullptr) return TABIT_EINVAL;
  const tabit::GemmConfig c = tabit::mx_config(index);
  *bm = c.bm;
  *bn = c.bn;
  return TABIT_OK;
}

int tabit_mxfp4_config_choose(int M, int N, int K, int num_cus) {
  if (M < 0 || N < 0 || K < 1) return TABIT_EINVAL;
  return tabit::mx_config_choose(M, N, K, num_cus);
}

int tabit_plane_config_info(int index, int* bm, int* bn, int* k_groups) {
  if (index < 0) return tabit::plane_config_count();
  if (index >= tabit::plane_config_count() || bm == nullptr || bn == nullptr) return TABIT_EINVAL;
  const tabit::GemmConfig c = tabit::plane_config(index);
  *bm = c.bm;
  *bn = c.bn;
  if (k_groups != nullptr) *k_groups = c.k_groups;
  return TABIT_OK;
}

int tabit_plane_config_choose(int M, int N, int K, int num_cus) {
  if (M < 0 || N < 0 || K < 1) return TABIT_EINVAL;
  return tabit::plane_config_choose(M, N, K, num_cus);
}

size_t tabit_mfma_probe_sink_ints(int num_cus) {
  return tabit::mfma_probe_sink_ints(num_cus > 0 ? num_cus : 256);
}

int tabit_mfma_peak_probe(tabit_ctx* ctx, int kind, int iters, int32_t* sink, size_t sink_ints,
                          double* ops_per_s, void* stream) {
  if (ctx == nullptr) return TABIT_EINVAL;
  if (kind != 0 && kind != 1) return fail(ctx, TABIT_EINVAL, "probe kind must be 0 or 1 (got %d)", kind);
  if (iters < 1 || iters > (1 << 24))
    return fail(ctx, TABIT_ERANGE, "iters must be in [1, 2^24] (got %d)", iters);
  if (sink == nullptr || ops_per_s == nullptr) return fail(ctx, TABIT_EINVAL, "null pointer");
  const int num_cus = tabit::device_num_cus();
  if (sink_ints < tabit::mfma_probe_sink_ints(num_cus))
    return fail(ctx, TABIT_ESHAPE, "sink holds %zu ints, %zu needed", sink_ints,
                tabit::mfma_probe_sink_ints(num_cus));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  double ops = 0.0;
  if (e == hipSuccess) ops = tabit::launch_mfma_probe(kind, iters, num_cus, sink, s, e0, e1, &e);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return hip_status(ctx, e, "mfma probe");
  *ops_per_s = ms > 0.0f ? ops / (ms * 1e-3) : 0.0;
  return TABIT_OK;
}

int tabit_gemm_config_choose(int M, int N, int K, int num_cus) {
  return tabit::gemm_config_choose(M, N, K, num_cus);
}

}  // extern "C"
