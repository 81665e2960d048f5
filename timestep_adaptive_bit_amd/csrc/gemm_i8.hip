// INT8 MFMA GEMMs for gfx950: the TASQ masked GEMM and its bit-plane form.
//
//   acc[m][n] = sum_k Xq[m][k] * ((Wq[n][k] >> kbits) << kbits)      (int32, exact)
//   Y[m][n]   = bf16_rne(((float)acc * sa[m]) * sw[n])
//
// TASQ (gist.science summary, section 2 "Metodologia"): one shared 8-bit
// weight buffer; the operational weight at (step, layer) drops the k least
// significant bits; the same kernel serves every k (k is a scalar argument).
// The bit-plane form evaluates sum_{b=k}^{7} c_b (Xq . W_b^T) with W_b bit b of
// the two's-complement byte (c_b = 2^b, sign plane -2^7): the activation
// fragment is loaded once per K-tile and reused against each retained plane,
// the analogue of the Temporal-Precision Engine keeping activation planes on
// chip and streaming only the selected weight planes.  A plane is the byte
// W & (1 << b) read as int8 ({0, 2^b}, or {0, -128} for b = 7), so its MFMA
// product is exactly c_b (Xq . W_b^T).
//
// Both operands are K-contiguous ([M][K] and [N][K]).  A workgroup computes a
// BM x BN tile with 2 x 2 waves; K advances in 128-byte steps through a
// double-buffered LDS tile (one barrier per step).  LDS rows are 128 bytes,
// 16-byte chunks XOR-swizzled by (row & 7) ^ ((row >> 3) & 1), which keeps
// both the staging writes and the MFMA operand reads (16 rows x one chunk per
// 16 lanes) free of bank conflicts.  The step's LSB mask is applied to the
// weight tile as it is staged into LDS.  The epilogue scales in fp32, rounds to
// bf16 and transposes through LDS so that global stores are 16-byte and
// row-contiguous.  Workgroup ids are remapped so that consecutive tiles stay on
// one XCD (dispatch round-robins workgroups over the 8 XCDs, each with its own
// L2), and tiles are walked in groups of 4 tile-rows for L2 reuse.
#include "tabit_internal.h"

namespace tabit {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int BK = 128;  // bytes (= int8 elements) of K per LDS stage

__device__ __forceinline__ int lds_off(int r, int c) {
  return r * BK + ((c ^ ((r & 7) ^ ((r >> 3) & 1))) << 4);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Logical tile of this workgroup: undo the round-robin XCD dispatch so that
// each XCD receives a contiguous range of logical ids, then walk tiles in
// groups of GROUP_M tile-rows (column-major within the group).
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

template <int BM, int BN, bool BITSERIAL>
__global__ void __launch_bounds__(256)
gemm_i8_kernel(const int8_t* __restrict__ A, const float* __restrict__ SA,
               const int8_t* __restrict__ B, const float* __restrict__ SB, int M, int N, int K,
               int kbits, uint16_t* __restrict__ Y, int32_t* __restrict__ ACC, int tiles_m,
               int tiles_n) {
  constexpr int NT = 256;
  constexpr int WM = 2, WN = 2;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_LD = BM * (BK / 16) / NT;
  constexpr int B_LD = BN * (BK / 16) / NT;
  constexpr int STAGE = (BM + BN) * BK;
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for 256 threads");
  static_assert(2 * STAGE >= BM * BN * 2, "epilogue tile must fit in the LDS stages");
  __shared__ __attribute__((aligned(16))) int8_t smem[2 * STAGE];

  int tm, tn;
  tile_coords<4>(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;

  const uint32_t m8 = (0xFFu << kbits) & 0xFFu;
  const int mask32 = (int)(m8 * 0x01010101u);

  v4i ra[A_LD], rb[B_LD];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int qd = i * NT + tid, r = qd >> 3, c = qd & 7;
      const int gm = m0 + r, gk = k0 + c * 16;
      ra[i] = (gm < M && gk < K) ? *reinterpret_cast<const v4i*>(A + (size_t)gm * K + gk)
                                 : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int qd = i * NT + tid, r = qd >> 3, c = qd & 7;
      const int gn = n0 + r, gk = k0 + c * 16;
      rb[i] = (gn < N && gk < K) ? *reinterpret_cast<const v4i*>(B + (size_t)gn * K + gk)
                                 : v4i{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
    int8_t* sa = smem + buf * STAGE;
    int8_t* sb = sa + BM * BK;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int qd = i * NT + tid;
      *reinterpret_cast<v4i*>(sa + lds_off(qd >> 3, qd & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int qd = i * NT + tid;
      v4i w = rb[i];
      if constexpr (!BITSERIAL) w &= mask32;  // TASQ LSB mask, applied while staging
      *reinterpret_cast<v4i*>(sb + lds_off(qd >> 3, qd & 7)) = w;
    }
  };

  v4i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const int8_t* sa = smem + cur * STAGE;
    const int8_t* sb = sa + BM * BK;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      v4i a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const v4i*>(sa + lds_off(wm * WTM + i * 16 + (lane & 15), c));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[j] = *reinterpret_cast<const v4i*>(sb + lds_off(wn * WTN + j * 16 + (lane & 15), c));
      if constexpr (!BITSERIAL) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
      } else {
        for (int p = 7; p >= kbits; --p) {
          const int pm = (int)(0x01010101u << p);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const v4i bp = b[j] & pm;
#pragma unroll
            for (int i = 0; i < FM; ++i)
              acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], bp, acc[i][j], 0, 0, 0);
          }
        }
      }
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  // MFMA 16x16 output layout: lane l, register r holds row 4*(l/16)+r, col l%16.
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
    float sa_r[FM][4], sb_c[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gm = row_base + i * 16 + r;
        sa_r[i][r] = gm < M ? SA[gm] : 0.0f;
      }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int gn = col_base + j * 16;
      sb_c[j] = gn < N ? SB[gn] : 0.0f;
    }
    // Each wave stages its WTM x WTN bf16 tile in its own LDS region; 16-byte
    // column chunks are XOR-swizzled by the row so the scattered 2-byte writes
    // and the row-contiguous 16-byte reads avoid bank conflicts.
    constexpr int CH = WTN / 8;  // 16-byte chunks per staged row
    uint16_t* st = reinterpret_cast<uint16_t*>(smem) + wave * WTM * WTN;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = i * 16 + 4 * (lane >> 4) + r;
          const int lc = j * 16 + (lane & 15);
          const float f = ((float)acc[i][j][r] * sa_r[i][r]) * sb_c[j];
          const int ch = (lc >> 3) ^ (lr & (CH - 1));
          st[lr * WTN + ch * 8 + (lc & 7)] = bf16_rne(f);
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
  float eff;  // relative MFMA efficiency used by the automatic choice
};
constexpr CfgDesc kCfgs[] = {
    {256, 256, 1.00f},
    {256, 128, 0.92f},
    {128, 128, 0.85f},
    {128, 64, 0.70f},
    {64, 64, 0.50f},
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

template <int BM, int BN>
hipError_t launch_cfg(bool bitserial, const int8_t* xq, const float* sa, const int8_t* wq,
                      const float* sw, int M, int N, int K, int kbits, uint16_t* y, int32_t* acc,
                      hipStream_t s) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int grid = tiles_m * tiles_n;
  if (bitserial)
    gemm_i8_kernel<BM, BN, true><<<grid, 256, 0, s>>>(xq, sa, wq, sw, M, N, K, kbits, y, acc,
                                                      tiles_m, tiles_n);
  else
    gemm_i8_kernel<BM, BN, false><<<grid, 256, 0, s>>>(xq, sa, wq, sw, M, N, K, kbits, y, acc,
                                                       tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

int gemm_config_count() { return kNumCfgs; }

GemmConfig gemm_config(int index) { return GemmConfig{kCfgs[index].bm, kCfgs[index].bn, 1}; }

int gemm_config_choose(int M, int N, int K, int num_cus) {
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

hipError_t launch_gemm_i8(int cfg, bool bitserial, const int8_t* xq, const float* sa,
                          const int8_t* wq, const float* sw, int M, int N, int K, int kbits,
                          uint16_t* y, int32_t* acc, hipStream_t stream) {
  switch (cfg) {
    case 0: return launch_cfg<256, 256>(bitserial, xq, sa, wq, sw, M, N, K, kbits, y, acc, stream);
    case 1: return launch_cfg<256, 128>(bitserial, xq, sa, wq, sw, M, N, K, kbits, y, acc, stream);
    case 2: return launch_cfg<128, 128>(bitserial, xq, sa, wq, sw, M, N, K, kbits, y, acc, stream);
    case 3: return launch_cfg<128, 64>(bitserial, xq, sa, wq, sw, M, N, K, kbits, y, acc, stream);
    default: return launch_cfg<64, 64>(bitserial, xq, sa, wq, sw, M, N, K, kbits, y, acc, stream);
  }
}

}  // namespace tabit
