// Activation / weight quantizers for gfx950.
//
// INT8: per row, unnormalized block Walsh-Hadamard transform (fp32; stages
// h = 1, 2, 4, ... so every output is a fixed sequence of IEEE additions),
// row absmax, one correctly rounded division r = 127/a, codes
// rint(y*r) clamped to +-127.  HQ-DM (gist.science summary, section 2.1):
// rotate X by a block-diagonal Hadamard, quantize XH, keep the Hadamard
// normalization in the fp scale.  Section 2.2: symmetric quantization.
//
// MXFP4: per block of 32, optional FWHT32, E8M0 scale 2^X with
// X = floor(log2 amax) - 2, E2M1 codes of y*2^-X rounded to nearest even.
// 6Bit-Diffusion (gist.science summary, section 2A): local block Hadamard
// before 4-bit quantization; OCP MX v1.0 defines the format.
//
// Data layout: the workgroup's rows are contiguous in memory, so the
// workgroup sees them as one flat run of 16-element chunks; chunk c of the run
// lives in thread (c mod NT), register slot (c / NT) for NT threads per workgroup.  Loads and stores are
// 16-byte, fully coalesced.  A Hadamard block of b elements spans b/16
// consecutive, aligned lanes, so the cross-lane FWHT stages are lane-XOR
// exchanges (DPP within a quad, ds_swizzle beyond).
#include "tabit_internal.h"

namespace tabit {
namespace {

constexpr int QT = 256;  // threads per workgroup of the MX quantizer

template <int MASK>
__device__ __forceinline__ float lane_xor(float v) {
  int i = __float_as_int(v);
  if constexpr (MASK == 1) {
    i = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (MASK == 2) {
    i = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else {
    i = __builtin_amdgcn_ds_swizzle(i, (MASK << 10) | 0x1F);  // bit mode: lane ^ MASK
  }
  return __int_as_float(i);
}

// One cross-lane butterfly stage: the lane holding the first element of each
// pair keeps first + second, its partner keeps first - second.
template <int MASK>
__device__ __forceinline__ void cross_stage(float (&v)[16], int lane) {
  const bool second = (lane & MASK) != 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float o = lane_xor<MASK>(v[e]);
    v[e] = second ? (o - v[e]) : (v[e] + o);
  }
}

// Unnormalized FWHT of one 16-element chunk, stages h = 1, 2, 4, 8 in registers,
// then h = 16, 32, 64 across lanes as the block size requires.
template <int B>
__device__ __forceinline__ void fwht_chunk(float (&v)[16], int lane) {
  if constexpr (B > 0) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 16; i += 2 * h) {
#pragma unroll
        for (int j = i; j < i + h; ++j) {
          const float a = v[j], b = v[j + h];
          v[j] = a + b;
          v[j + h] = a - b;
        }
      }
    }
    if constexpr (B >= 32) cross_stage<1>(v, lane);
    if constexpr (B >= 64) cross_stage<2>(v, lane);
    if constexpr (B >= 128) cross_stage<4>(v, lane);
  }
}

__device__ __forceinline__ void load_chunk(const uint16_t* p, float (&v)[16]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  const uint4 a = q[0], b = q[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t tile_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack4_i8(float a, float b, float c, float d, float r) {
  const int qa = (int)__builtin_amdgcn_fmed3f(rintf(a * r), -127.0f, 127.0f);
  const int qb = (int)__builtin_amdgcn_fmed3f(rintf(b * r), -127.0f, 127.0f);
  const int qc = (int)__builtin_amdgcn_fmed3f(rintf(c * r), -127.0f, 127.0f);
  const int qd = (int)__builtin_amdgcn_fmed3f(rintf(d * r), -127.0f, 127.0f);
  return (uint32_t)(qa & 0xFF) | ((uint32_t)(qb & 0xFF) << 8) | ((uint32_t)(qc & 0xFF) << 16) |
         ((uint32_t)qd << 24);
}

// Row of a chunk index (c < 2^16, cr < 2^12): float estimate, then exact fix-up.
__device__ __forceinline__ int row_of(int c, int cr, float inv_cr) {
  int r = (int)((float)c * inv_cr);
  if (r * cr > c) --r;
  if ((r + 1) * cr <= c) ++r;
  return r;
}

// GELU, tanh form: 0.5 x (1 + tanh(u)) = x sigma(z) with z = 2u =
// x (k1 + k3 x^2), k1 = 2 sqrt(2/pi), k3 = 0.044715 k1, sigma(z) = 1/(1 + e^-z).
// sigma comes from t = e^-|z| (in (0, 1], never overflows): 1/(1 + t) for
// z >= 0, t/(1 + t) for z < 0, with the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32).  In fp32 the result is within 16 ulp (z >= 0) or
// (16|z| + 24) ulp (z < 0) of the exact GELU, ulp = 2^-24 relative; results
// of magnitude below 2^-100 become 0 (the deep negative tail, where no fp32
// evaluation keeps relative accuracy).  +-inf in z gives 0 or x, never NaN.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float z = x * (0x1.988454p+0f + 0x1.2444f2p-4f * (x * x));
  const float t = __builtin_amdgcn_exp2f(-fabsf(z) * 0x1.715476p+0f);
  const float s = __builtin_amdgcn_rcpf(1.0f + t);
  const float g = x * (z >= 0.0f ? s : t * s);
  return fabsf(g) < 0x1p-100f ? 0.0f : g;
}

enum QuantMode { Q_PLAIN = 0, Q_HQDM = 1, Q_GELU = 2 };

// MODE = Q_GELU: each input element becomes bf16(gelu(x)) first (the MLP's
// activation folded into the quantizer of the down projection's input).
// MODE = Q_PLAIN: codes of the rotated row.  MODE = Q_HQDM (HQ-DM single Hadamard):
// the codes are rotated back by the same block FWHT -- integers up to 127 b in
// magnitude, exact in fp32 -- and written as two int8 planes Z = 128 hi + lo
// (hi = floor(Z / 128) to q, lo in [0, 127] to q_lo).
// ONE: the workgroup holds a single row; its absmax is then a butterfly over
// each wave's lanes and one value per wave in LDS (one barrier), instead of
// LDS atomics per row (max is exact in any order, so the codes are the same).
template <int B, int NT, int CPT, int MODE, bool ONE>
__global__ void __launch_bounds__(NT)
quant_int8_kernel(const uint16_t* __restrict__ x, int M, int K, int rows_per_wg, float scale_div,
                  int8_t* __restrict__ q, float* __restrict__ scale, const uint8_t* __restrict__ gate,
                  int8_t* __restrict__ q_lo) {
  if (gate != nullptr && *gate != 0) return;   // device-selected format is not INT8
  __shared__ unsigned s_amax[ONE ? 1 : NT * CPT / 2];
  __shared__ float s_r[ONE ? 1 : NT * CPT / 2];
  __shared__ float s_wmax[NT / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int r0 = blockIdx.x * rows_per_wg;
  const int rows = min(rows_per_wg, M - r0);
  const int cr = K >> 4;
  const int nchunks = rows * cr;
  const float inv_cr = 1.0f / (float)cr;
  const size_t base = (size_t)r0 * (size_t)K;

  float v[CPT][16];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = i * NT + tid;
    if (c < nchunks) {
      load_chunk(x + base + (size_t)c * 16, v[i]);
      if constexpr (MODE == Q_GELU) {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[i][e] = __uint_as_float((uint32_t)tile_bf16(gelu_tanh(v[i][e])) << 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[i][e] = 0.0f;
    }
  }
  if constexpr (!ONE)
    for (int t = tid; t < rows; t += NT) s_amax[t] = 0u;
#pragma unroll
  for (int i = 0; i < CPT; ++i) fwht_chunk<B>(v[i], lane);

  float r_one = 0.0f;   // 127 / absmax of the row (ONE)
  if constexpr (ONE) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if (i * NT + tid < nchunks)
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[i][e]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (lane == 0) s_wmax[tid >> 6] = m;
    __syncthreads();
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) a = fmaxf(a, s_wmax[w]);
    r_one = a > 0.0f ? 127.0f / a : 0.0f;
    if (tid == 0) scale[r0] = (a / 127.0f) / scale_div;
  } else {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = i * NT + tid;
      if (c < nchunks) {
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[i][e]));
        // non-negative floats order like their bit patterns
        atomicMax(&s_amax[row_of(c, cr, inv_cr)], __float_as_uint(m));
      }
    }
    __syncthreads();
    for (int t = tid; t < rows; t += NT) {
      const float a = __uint_as_float(s_amax[t]);
      s_r[t] = a > 0.0f ? 127.0f / a : 0.0f;
      scale[r0 + t] = (a / 127.0f) / scale_div;
    }
    __syncthreads();
  }
  auto r_of = [&](int c) { return ONE ? r_one : s_r[row_of(c, cr, inv_cr)]; };

  if constexpr (MODE != Q_HQDM) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = i * NT + tid;
      if (c < nchunks) {
        const float r = r_of(c);
        uint4 o;
        o.x = pack4_i8(v[i][0], v[i][1], v[i][2], v[i][3], r);
        o.y = pack4_i8(v[i][4], v[i][5], v[i][6], v[i][7], r);
        o.z = pack4_i8(v[i][8], v[i][9], v[i][10], v[i][11], r);
        o.w = pack4_i8(v[i][12], v[i][13], v[i][14], v[i][15], r);
        *reinterpret_cast<uint4*>(q + base + (size_t)c * 16) = o;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = i * NT + tid;
      const float r = c < nchunks ? r_of(c) : 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e)   // the codes, as pack4_i8 forms them
        v[i][e] = __builtin_amdgcn_fmed3f(rintf(v[i][e] * r), -127.0f, 127.0f);
      fwht_chunk<B>(v[i], lane);      // every lane: the cross-lane stages need all of them
      if (c < nchunks) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          hw[d] = 0u;
          lw[d] = 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int z = (int)v[i][4 * d + e];
            hw[d] |= (uint32_t)((z >> 7) & 0xFF) << (8 * e);
            lw[d] |= (uint32_t)(z & 127) << (8 * e);
          }
        }
        *reinterpret_cast<uint4*>(q + base + (size_t)c * 16) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4*>(q_lo + base + (size_t)c * 16) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
    }
  }
}

// E2M1 codes of a and b (already scaled by 2^-X) in the low and high nibble of
// a byte: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even mantissa
// bit, saturating at 6.  gfx950's packed FP4 conversion rounds and saturates
// exactly so (checked on the device against the comparison-chain definition
// over [-10, 10] in steps of 1/400, every tie, +-0 and subnormals; its scale
// operand divides, and 1.0 leaves the values as they are).
__device__ __forceinline__ uint32_t e2m1_pair(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

// The conversion keeps the sign of a value that rounds to zero (code 8); the
// format's convention here encodes -0 as +0: clear bit 3 of every nibble whose
// magnitude bits are zero (adding 7 to 3 magnitude bits carries into bit 3
// exactly when they are nonzero, and never out of the nibble).
__device__ __forceinline__ uint32_t drop_negative_zero(uint32_t x) {
  const uint32_t mag = x & 0x77777777u;
  return mag | (x & ((mag + 0x77777777u) & 0x88888888u));
}

// GELU: each input element becomes bf16(gelu(x)) first (the MLP's activation
// folded into the quantizer of the down projection's input, as in
// quant_int8_kernel's Q_GELU mode).
template <int B, int CPT, bool GELU>
__global__ void __launch_bounds__(QT)
quant_mx_kernel(const uint16_t* __restrict__ x, long long nchunks, uint8_t* __restrict__ qf,
                uint8_t* __restrict__ e8, const uint8_t* __restrict__ gate) {
  if (gate != nullptr && *gate != 1) return;   // device-selected format is not MXFP4
  const int tid = threadIdx.x;
  const int lane = tid & 63;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const long long c = ((long long)blockIdx.x * CPT + i) * QT + tid;
    const bool valid = c < nchunks;
    float v[16];
    if (valid) {
      load_chunk(x + c * 16, v);
      if constexpr (GELU) {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = __uint_as_float((uint32_t)tile_bf16(gelu_tanh(v[e])) << 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = 0.0f;
    }
    fwht_chunk<B>(v, lane);
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[e]));
    m = fmaxf(m, lane_xor<1>(m));  // the 32-block spans this lane and its XOR-1 partner
    const uint32_t bits = __float_as_uint(m);
    const int ex = (int)((bits >> 23) & 0xFFu);
    int X;
    if (m == 0.0f) {
      X = 0;
    } else if (ex == 0) {
      X = -127;  // subnormal amax: floor(log2) <= -127
    } else {
      X = min(max(ex - 127 - 2, -127), 127);
    }
    const float inv = __uint_as_float((uint32_t)(127 - X) << 23);  // 2^-X, exact
    uint32_t lo = 0u, hi = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= e2m1_pair(v[2 * e] * inv, v[2 * e + 1] * inv) << (8 * e);
      hi |= e2m1_pair(v[8 + 2 * e] * inv, v[8 + 2 * e + 1] * inv) << (8 * e);
    }
    lo = drop_negative_zero(lo);
    hi = drop_negative_zero(hi);
    if (valid) {
      *reinterpret_cast<uint2*>(qf + c * 8) = make_uint2(lo, hi);
      if ((c & 1) == 0) e8[c >> 1] = (uint8_t)(X + 127);
    }
  }
}

template <int B, int MODE>
hipError_t dispatch_int8(int nt, int cpt, int grid, int rows, const uint16_t* x, int M, int K,
                         float scale_div, int8_t* q, float* scale, hipStream_t s, const uint8_t* gate,
                         int8_t* q_lo) {
#define TABIT_Q(NT_, CPT_, ONE_)                                                                \
  if (nt == NT_ && cpt == CPT_ && (rows == 1) == ONE_) {                                        \
    quant_int8_kernel<B, NT_, CPT_, MODE, ONE_><<<grid, NT_, 0, s>>>(x, M, K, rows, scale_div, q, \
                                                                   scale, gate, q_lo);          \
    return hipGetLastError();                                                                   \
  }
  TABIT_Q(256, 1, false) TABIT_Q(64, 1, true) TABIT_Q(128, 1, true) TABIT_Q(192, 1, true) TABIT_Q(256, 1, true) TABIT_Q(320, 1, true)
  TABIT_Q(384, 1, true) TABIT_Q(448, 1, true) TABIT_Q(512, 1, true) TABIT_Q(1024, 1, true)
  TABIT_Q(1024, 2, true)
#undef TABIT_Q
  return hipErrorInvalidValue;
}

}  // namespace

namespace {

// Workgroup shape: one 16-element chunk per thread.  A row of up to 512
// chunks gets a workgroup of its own sized to the next multiple of 64 threads
// when that keeps at least as large a share of the threads busy as packing
// whole rows into 256 threads, else it shares a 256-thread workgroup (rows of
// up to 32 chunks always do): 320 threads for the 288 chunks of K = 4608
// (13.1 vs 14.0 us at 4096 rows with 512, 13.6 with two rows in 576), 128 for
// the 120 of K = 1920 (17.9 vs 19.0 us at 17776 rows), three rows in 256 for
// the 72 of K = 1152 (4.5 vs 4.8 us hot with one row in 128).  Longer rows
// take 1024 threads, two chunks per thread past 1024 chunks.  Small workgroups with few registers outnumber the resident slots,
// so reads of late workgroups overlap the stores of early ones; on MI355X this
// beat fuller multi-row, multi-chunk shapes by 7-32% at the workloads' sizes.
template <int MODE>
hipError_t launch_int8_rows(const uint16_t* x, int M, int K, int had_block, float scale_div,
                            int8_t* q, float* scale, hipStream_t stream, const uint8_t* gate,
                            int8_t* q_lo) {
  if (M <= 0) return hipSuccess;
  const int cr = K / 16;
  int nt = 1024, cpt = 1;
  if (cr <= 512) {
    const int one = (cr + 63) / 64 * 64;   // a workgroup of its own, next multiple of 64 threads
    const int multi = 256 / cr * cr;       // chunks of whole rows a 256-thread workgroup holds
    nt = cr > 32 && cr * 256 >= multi * one ? one : 256;   // the shape that keeps more threads busy
  }
  else if (cr > 1024) cpt = 2;
  const int rows = (nt * cpt) / cr;
  const int grid = (M + rows - 1) / rows;
  switch (had_block) {
    case 0: return dispatch_int8<0, MODE>(nt, cpt, grid, rows, x, M, K, scale_div, q, scale, stream, gate, q_lo);
    case 32: return dispatch_int8<32, MODE>(nt, cpt, grid, rows, x, M, K, scale_div, q, scale, stream, gate, q_lo);
    case 64: return dispatch_int8<64, MODE>(nt, cpt, grid, rows, x, M, K, scale_div, q, scale, stream, gate, q_lo);
    default: return dispatch_int8<128, MODE>(nt, cpt, grid, rows, x, M, K, scale_div, q, scale, stream, gate, q_lo);
  }
}

}  // namespace

hipError_t launch_quant_int8(const uint16_t* x, int M, int K, int had_block, float scale_div,
                             int8_t* q, float* scale, hipStream_t stream, const uint8_t* gate) {
  return launch_int8_rows<Q_PLAIN>(x, M, K, had_block, scale_div, q, scale, stream, gate, nullptr);
}

hipError_t launch_quant_gelu_int8(const uint16_t* x, int M, int K, int had_block, int8_t* q,
                                  float* scale, hipStream_t stream, const uint8_t* gate) {
  return launch_int8_rows<Q_GELU>(x, M, K, had_block, 1.0f, q, scale, stream, gate, nullptr);
}

hipError_t launch_quant_hqdm(const uint16_t* x, int M, int K, int had_block, int8_t* q_hi,
                             int8_t* q_lo, float* scale, hipStream_t stream, const uint8_t* gate) {
  const float div = (float)(had_block > 0 ? had_block : 1);   // X ~ (s_a / b) Z
  return launch_int8_rows<Q_HQDM>(x, M, K, had_block, div, q_hi, scale, stream, gate, q_lo);
}

namespace {

template <bool GELU>
hipError_t launch_mx(const uint16_t* x, int M, int K, int had_block, uint8_t* q_fp4,
                     uint8_t* e8m0, hipStream_t stream, const uint8_t* gate) {
  if (M <= 0) return hipSuccess;
  constexpr int CPT = 1;   // one chunk per thread: 7-36% faster than 2-8 on MI355X
  const long long nchunks = (long long)M * K / 16;
  const long long per_wg = (long long)QT * CPT;
  const int grid = (int)((nchunks + per_wg - 1) / per_wg);
  if (had_block == 32) {
    quant_mx_kernel<32, CPT, GELU><<<grid, QT, 0, stream>>>(x, nchunks, q_fp4, e8m0, gate);
  } else {
    quant_mx_kernel<0, CPT, GELU><<<grid, QT, 0, stream>>>(x, nchunks, q_fp4, e8m0, gate);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_mx(const uint16_t* x, int M, int K, int had_block, uint8_t* q_fp4,
                           uint8_t* e8m0, hipStream_t stream, const uint8_t* gate) {
  return launch_mx<false>(x, M, K, had_block, q_fp4, e8m0, stream, gate);
}

hipError_t launch_quant_gelu_mx(const uint16_t* x, int M, int K, int had_block, uint8_t* q_fp4,
                                uint8_t* e8m0, hipStream_t stream, const uint8_t* gate) {
  return launch_mx<true>(x, M, K, had_block, q_fp4, e8m0, stream, gate);
}

}  // namespace tabit
