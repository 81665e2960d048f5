// Internal declarations shared by the HIP translation units of libtabit.
// Not part of the public ABI (see include/tabit.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <map>
#include <string>
#include <tuple>
#include <vector>

namespace tabit {

// ---------------------------------------------------------------- quantizers
// Per-row INT8 quantization with an optional block FWHT (activations and
// weights).  scale_div divides the per-row scale a/127 (1 for activations,
// max(b, 1) for weights).
// gate (optional, every launcher below): device byte holding the format the
// caller's schedule selected; a kernel whose format differs returns at once.
hipError_t launch_quant_int8(const uint16_t* x, int M, int K, int had_block, float scale_div,
                             int8_t* q, float* scale, hipStream_t stream,
                             const uint8_t* gate = nullptr);

// Quantizer of the MLP down projection's input with the GELU (tanh form)
// folded in: codes of blockFWHT_b(bf16(gelu(x))).
hipError_t launch_quant_gelu_int8(const uint16_t* x, int M, int K, int had_block, int8_t* q,
                                  float* scale, hipStream_t stream, const uint8_t* gate = nullptr);

// HQ-DM single Hadamard: codes of the rotated row rotated back, Z = 128 hi + lo
// as two int8 planes; scale = (a / 127) / max(b, 1).
hipError_t launch_quant_hqdm(const uint16_t* x, int M, int K, int had_block, int8_t* q_hi,
                             int8_t* q_lo, float* scale, hipStream_t stream,
                             const uint8_t* gate = nullptr);

// MXFP4 quantization (block 32, optional FWHT32).
hipError_t launch_quant_mx(const uint16_t* x, int M, int K, int had_block,
                           uint8_t* q_fp4, uint8_t* e8m0, hipStream_t stream,
                           const uint8_t* gate = nullptr);

// MXFP4 quantization of bf16(gelu(x)) (the MLP's GELU folded in).
hipError_t launch_quant_gelu_mx(const uint16_t* x, int M, int K, int had_block,
                                uint8_t* q_fp4, uint8_t* e8m0, hipStream_t stream,
                                const uint8_t* gate = nullptr);

// ---------------------------------------------------------------- INT8 GEMM
struct GemmConfig {
  int bm, bn, k_groups;   // wave groups splitting one tile's K stages (1 = none)
};
int gemm_config_count();
GemmConfig gemm_config(int index);
int gemm_config_choose(int M, int N, int K, int num_cus);

// ev0 / ev1 (optional): events stamped with this GEMM kernel's start and stop.
hipError_t launch_gemm_i8(int cfg, bool bitserial, const int8_t* xq, const float* sa,
                          const int8_t* wq, const float* sw, int M, int N, int K, int kbits,
                          uint16_t* y, int32_t* acc, hipStream_t stream,
                          hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr,
                          const uint8_t* gate = nullptr);

// ---------------------------------------------------------------- MXFP4 GEMM
int mx_config_count();
GemmConfig mx_config(int index);
int mx_config_choose(int M, int N, int K, int num_cus);

hipError_t launch_gemm_mxfp4(int cfg, const uint8_t* xq, const uint8_t* xe, const uint8_t* wq,
                             const uint8_t* we, int M, int N, int K, float out_scale,
                             uint16_t* y, float* acc, hipStream_t stream,
                             hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr,
                             const uint8_t* gate = nullptr);

// ---------------------------------------------------------------- plane-major storage
// uint32 P[8][ceil(K/128)][N][4]: word P[b][s][n][j] holds bit b of
// W[n][128s + 32j + i] at bit 8*(i % 4) + i / 4; words past K are zero.
size_t planes_bytes(int N, int K);
hipError_t launch_pack_planes(const int8_t* wq, int N, int K, uint32_t* planes, hipStream_t s);
int plane_config_count();
GemmConfig plane_config(int index);
int plane_config_choose(int M, int N, int K, int num_cus);
hipError_t launch_gemm_planes(int cfg, const int8_t* xq, const float* sa, const uint32_t* wp,
                              const float* sw, int M, int N, int K, int kbits, uint16_t* y,
                              int32_t* acc, hipStream_t stream, hipEvent_t ev0 = nullptr,
                              hipEvent_t ev1 = nullptr, const uint8_t* gate = nullptr);

// ---------------------------------------------------------------- HQ-DM single-Hadamard GEMM
int hqdm_config_count();
GemmConfig hqdm_config(int index);
int hqdm_config_choose(int M, int N, int K, int num_cus);
hipError_t launch_gemm_hqdm(int cfg, const int8_t* xh, const int8_t* xl, const float* sa,
                            const int8_t* wq, const float* sw, int M, int N, int K, int kbits,
                            uint16_t* y, long long* acc, hipStream_t stream,
                            hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// ---------------------------------------------------------------- DMPQ selector
// Gamma = sum |out - in| / sum |in| of a block's hidden states in the fixed
// fp64 order; fmt[l] = Gamma > theta[l] ? INT8 : MXFP4.  rows: M x 2 doubles.
size_t dmpq_workspace_bytes(int M);
hipError_t launch_dmpq_select(const uint16_t* xin, const uint16_t* xout, int M, int H, double* rows,
                              const float* theta, int n_layers, uint8_t* fmt, double* gamma,
                              hipStream_t s);

// ---------------------------------------------------------------- matrix-core rate probe
// kind 0: INT8 32x32x32 MFMA; kind 1: FP4 32x32x64 scaled MFMA.  sink holds
// mfma_probe_sink_ints(num_cus) ints.  Returns the operations the launch performs.
size_t mfma_probe_sink_ints(int num_cus);
double launch_mfma_probe(int kind, int iters, int num_cus, int* sink, hipStream_t s,
                         hipEvent_t ev0, hipEvent_t ev1, hipError_t* err);

// Compute units of the current device (cached per device id).
int device_num_cus();

}  // namespace tabit

struct tabit_ctx {
  std::string err;
  int steps = 0;
  int layers = 0;
  std::vector<uint8_t> k_bits;
  std::vector<uint8_t> fmt;
  int force_gemm_cfg = -1;
  int force_mx_cfg = -1;
  int force_plane_cfg = -1;
  int force_hqdm_cfg = -1;
  // autotuned tile configuration per (path, M, N, K); path 2 = MXFP4, 3 = plane-major
  std::map<std::tuple<int, int, int, int>, int> tuned;

  int tuned_cfg(int path, int M, int N, int K) const {
    auto it = tuned.find(std::make_tuple(path, M, N, K));
    return it == tuned.end() ? -1 : it->second;
  }
};
