// MXFP4 (W4A4) GEMM for gfx950 on the block-scaled FP4 matrix cores.
//
//   acc[m][n] = sum_j 2^(xe[m][j]-127) 2^(we[n][j]-127) sum_{i in block j} e2m1(x) e2m1(w)
//   Y = bf16_rne(acc * out_scale)
//
// 6Bit-Diffusion (gist.science summary, section 2A): stable layers run their
// linear in a 4-bit format after a local block Hadamard; the page's NVFP4 is
// replaced by OCP MXFP4, the 4-bit format gfx950's matrix cores consume
// natively (32-element blocks, E8M0 scales applied inside the MFMA).
//
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1: lane l supplies
// 16 bytes = 32 consecutive K elements of row (l % 16) -- exactly one MX block
// -- and that block's E8M0 byte as its scale operand.  Tiling follows the INT8
// GEMM: 2 x 2 waves, 128-byte (256-element) K stages, double-buffered LDS with
// the same XOR swizzle; the stage's 8 scale bytes per row are staged next to
// the data tile.
#include "tabit_internal.h"

namespace tabit {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BKB = 128;  // bytes of packed K per stage (256 elements)
constexpr int SPR = 8;    // scale bytes per row per stage

__device__ __forceinline__ int lds_off(int r, int c) {
  return r * BKB + ((c ^ ((r & 7) ^ ((r >> 3) & 1))) << 4);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int G = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, j = bid >> 3;
  const int q = G >> 3, rem = G & 7;
  const int lin = xcd * q + min(xcd, rem) + j;
  const int per_group = GROUP_M * tiles_n;
  const int g = lin / per_group;
  const int first_m = g * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in_g = lin - g * per_group;
  tm = first_m + in_g % gsz;
  tn = in_g / gsz;
}

template <int BM, int BN>
__global__ void __launch_bounds__(256)
gemm_mxfp4_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ AE,
                  const uint8_t* __restrict__ B, const uint8_t* __restrict__ BE, int M, int N,
                  int K, float out_scale, uint16_t* __restrict__ Y, float* __restrict__ ACC,
                  int tiles_m, int tiles_n) {
  constexpr int NT = 256;
  constexpr int WM = 2, WN = 2;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_LD = BM * (BKB / 16) / NT;
  constexpr int B_LD = BN * (BKB / 16) / NT;
  constexpr int DATA = (BM + BN) * BKB;
  constexpr int STAGE = DATA + (BM + BN) * SPR;
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for 256 threads");
  static_assert(2 * STAGE >= BM * BN * 2, "epilogue tile must fit in the LDS stages");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  int tm, tn;
  tile_coords<4>(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int KB = K >> 1;        // packed bytes per row
  const int KS = K >> 5;        // scale bytes per row

  v4i ra[A_LD], rb[B_LD];
  uint8_t rsa[(BM * SPR + NT - 1) / NT], rsb[(BN * SPR + NT - 1) / NT];
  constexpr int SA_LD = (BM * SPR + NT - 1) / NT, SB_LD = (BN * SPR + NT - 1) / NT;
  auto gload = [&](int kt) {
    const int kb0 = kt * BKB;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int qd = i * NT + tid, r = qd >> 3, c = qd & 7;
      const int gm = m0 + r, gk = kb0 + c * 16;
      ra[i] = (gm < M && gk < KB) ? *reinterpret_cast<const v4i*>(A + (size_t)gm * KB + gk)
                                  : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int qd = i * NT + tid, r = qd >> 3, c = qd & 7;
      const int gn = n0 + r, gk = kb0 + c * 16;
      rb[i] = (gn < N && gk < KB) ? *reinterpret_cast<const v4i*>(B + (size_t)gn * KB + gk)
                                  : v4i{0, 0, 0, 0};
    }
    const int ks0 = kt * SPR;
#pragma unroll
    for (int i = 0; i < SA_LD; ++i) {
      const int qd = i * NT + tid, r = qd / SPR, j = qd % SPR;
      const int gm = m0 + r, gs = ks0 + j;
      rsa[i] = (r < BM && gm < M && gs < KS) ? AE[(size_t)gm * KS + gs] : (uint8_t)127;
    }
#pragma unroll
    for (int i = 0; i < SB_LD; ++i) {
      const int qd = i * NT + tid, r = qd / SPR, j = qd % SPR;
      const int gn = n0 + r, gs = ks0 + j;
      rsb[i] = (r < BN && gn < N && gs < KS) ? BE[(size_t)gn * KS + gs] : (uint8_t)127;
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* sa = smem + buf * STAGE;
    uint8_t* sb = sa + BM * BKB;
    uint8_t* ssa = sa + DATA;
    uint8_t* ssb = ssa + BM * SPR;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int qd = i * NT + tid;
      *reinterpret_cast<v4i*>(sa + lds_off(qd >> 3, qd & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int qd = i * NT + tid;
      *reinterpret_cast<v4i*>(sb + lds_off(qd >> 3, qd & 7)) = rb[i];
    }
#pragma unroll
    for (int i = 0; i < SA_LD; ++i) {
      const int qd = i * NT + tid;
      if (qd < BM * SPR) ssa[qd] = rsa[i];
    }
#pragma unroll
    for (int i = 0; i < SB_LD; ++i) {
      const int qd = i * NT + tid;
      if (qd < BN * SPR) ssb[qd] = rsb[i];
    }
  };

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nk = (KB + BKB - 1) / BKB;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* sa = smem + cur * STAGE;
    const uint8_t* sb = sa + BM * BKB;
    const uint8_t* ssa = sa + DATA;
    const uint8_t* ssb = ssa + BM * SPR;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      v4i a[FM], b[FN];
      int ea[FM], eb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * 16 + (lane & 15);
        a[i] = *reinterpret_cast<const v4i*>(sa + lds_off(r, c));
        ea[i] = ssa[r * SPR + c];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WTN + j * 16 + (lane & 15);
        b[j] = *reinterpret_cast<const v4i*>(sb + lds_off(r, c));
        eb[j] = ssb[r * SPR + c];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const v8i a8 = {a[i][0], a[i][1], a[i][2], a[i][3], 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v8i b8 = {b[j][0], b[j][1], b[j][2], b[j][3], 0, 0, 0, 0};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[i][j], 4, 4, 0,
                                                                        ea[i], 0, eb[j]);
        }
      }
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  const int row_base = m0 + wm * WTM + 4 * (lane >> 4);
  const int col_base = n0 + wn * WTN + (lane & 15);
  if (ACC != nullptr) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gm = row_base + i * 16 + r, gn = col_base + j * 16;
          if (gm < M && gn < N) ACC[(size_t)gm * N + gn] = acc[i][j][r];
        }
  }
  if (Y != nullptr) {
    constexpr int CH = WTN / 8;
    uint16_t* st = reinterpret_cast<uint16_t*>(smem) + wave * WTM * WTN;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = i * 16 + 4 * (lane >> 4) + r;
          const int lc = j * 16 + (lane & 15);
          const int ch = (lc >> 3) ^ (lr & (CH - 1));
          st[lr * WTN + ch * 8 + (lc & 7)] = bf16_rne(acc[i][j][r] * out_scale);
        }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < WTM * CH / 64; ++it) {
      const int idx = it * 64 + lane;
      const int lr = idx / CH, ch = idx % CH;
      const int gm = m0 + wm * WTM + lr, gn = n0 + wn * WTN + ch * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(st + lr * WTN + ((ch ^ (lr & (CH - 1))) * 8));
      if (gm < M && gn < N) *reinterpret_cast<uint4*>(Y + (size_t)gm * N + gn) = v;
    }
  }
}

struct CfgDesc {
  int bm, bn;
  float eff;
};
constexpr CfgDesc kCfgs[] = {
    {256, 256, 1.00f},
    {128, 128, 0.85f},
    {64, 64, 0.50f},
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

template <int BM, int BN>
hipError_t launch_cfg(const uint8_t* xq, const uint8_t* xe, const uint8_t* wq, const uint8_t* we,
                      int M, int N, int K, float out_scale, uint16_t* y, float* acc,
                      hipStream_t s) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  gemm_mxfp4_kernel<BM, BN><<<tiles_m * tiles_n, 256, 0, s>>>(xq, xe, wq, we, M, N, K, out_scale,
                                                              y, acc, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

int mx_config_count() { return kNumCfgs; }

GemmConfig mx_config(int index) { return GemmConfig{kCfgs[index].bm, kCfgs[index].bn, 1}; }

int mx_config_choose(int M, int N, int K, int num_cus) {
  (void)K;
  if (num_cus <= 0) num_cus = 256;
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < kNumCfgs; ++i) {
    const long long tiles = (long long)((M + kCfgs[i].bm - 1) / kCfgs[i].bm) *
                            ((N + kCfgs[i].bn - 1) / kCfgs[i].bn);
    const long long per_cu = (tiles + num_cus - 1) / num_cus;
    const double cost = (double)per_cu * kCfgs[i].bm * kCfgs[i].bn / kCfgs[i].eff;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = i;
    }
  }
  return best;
}

hipError_t launch_gemm_mxfp4(int cfg, const uint8_t* xq, const uint8_t* xe, const uint8_t* wq,
                             const uint8_t* we, int M, int N, int K, float out_scale, uint16_t* y,
                             float* acc, hipStream_t stream) {
  switch (cfg) {
    case 0: return launch_cfg<256, 256>(xq, xe, wq, we, M, N, K, out_scale, y, acc, stream);
    case 1: return launch_cfg<128, 128>(xq, xe, wq, we, M, N, K, out_scale, y, acc, stream);
    default: return launch_cfg<64, 64>(xq, xe, wq, we, M, N, K, out_scale, y, acc, stream);
  }
}

}  // namespace tabit
