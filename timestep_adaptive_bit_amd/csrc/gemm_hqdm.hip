// HQ-DM single-Hadamard GEMM (gist.science summary of HQ-DM, section 2.1):
// only the activations are rotated; inference recovers them through the
// orthogonality of H, X_hat = (s_a / b) Z with Z = (XH)_int H, and multiplies
// them with the untransformed weights.  Z (|Z| <= 127 b) arrives as two int8
// planes, Z = 128 hi + lo, so the integer core is two INT8 products against
// the same TASQ-truncated weight tile (TASQ summary, section 2):
//
//   acc_hi = hi . W_k^T,  acc_lo = lo . W_k^T          (int32, exact)
//   v      = 128 acc_hi + acc_lo                        (fp64, exact: |v| < 2^53)
//   Y      = bf16_rne(((float)v * s_a') * s_w)           (s_a' = s_a / b)
//
// The tile skeleton is the masked GEMM's (LDS-DMA stages of 128-byte rows,
// XOR swizzle, v_mfma_i32_32x32x32_i8, LSB mask on the weight fragments), with
// both activation planes staged next to the weights; each masked weight
// fragment feeds the MFMAs of both planes.
#include "tabit_internal.h"
#include "tile_common.h"

namespace tabit {
namespace {

using tile::v4i;
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int RB = 128;

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM* WN * 64)
gemm_hqdm_kernel(const int8_t* __restrict__ AH, const int8_t* __restrict__ AL,
                 const float* __restrict__ SA, const int8_t* __restrict__ B,
                 const float* __restrict__ SB, int M, int N, int K, int kbits,
                 uint16_t* __restrict__ Y, long long* __restrict__ ACC, int tiles_m, int tiles_n) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int KS = RB / 32;
  constexpr int SA_BYTES = BM * RB, SB_BYTES = BN * RB;
  constexpr int STAGE = 2 * SA_BYTES + SB_BYTES;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold whole 32x32 blocks");
  static_assert(2 * STAGE >= BM * BN * 2, "epilogue tile must fit in the LDS stages");
  __shared__ __attribute__((aligned(1024))) int8_t smem[2 * STAGE];

  int tm, tn;
  tile::tile_coords<4>(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
  const auto rsh = tile::make_rsrc(AH, (unsigned)M * (unsigned)K);
  const auto rsl = tile::make_rsrc(AL, (unsigned)M * (unsigned)K);
  const auto rsb = tile::make_rsrc(B, (unsigned)N * (unsigned)K);
  const uint32_t m8 = (0xFFu << kbits) & 0xFFu;
  const int mask32 = (int)(m8 * 0x01010101u);

  v16i ah[FM][FN], al[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      ah[i][j] = v16i{};
      al[i][j] = v16i{};
    }

  const int ra0 = wm * WTM + (lane & 31), rb0 = wn * WTN + (lane & 31);
  const int khalf = lane >> 5;
  const int nk = (K + RB - 1) / RB;
  auto issue = [&](int kt) {
    int8_t* dst = smem + (kt & 1) * STAGE;
    tile::dma_stage<BM, NW, RB>(rsh, dst, m0, rows_a, K, kt * RB, wave, lane);
    tile::dma_stage<BM, NW, RB>(rsl, dst + SA_BYTES, m0, rows_a, K, kt * RB, wave, lane);
    tile::dma_stage<BN, NW, RB>(rsb, dst + 2 * SA_BYTES, n0, rows_b, K, kt * RB, wave, lane);
  };
  issue(0);
  for (int kt = 0; kt < nk; ++kt) {
    tile::wait_vmcnt<0>();
    __syncthreads();   // stage kt visible to all; stage kt-1's buffer is free
    if (kt + 1 < nk) issue(kt + 1);
    const int8_t* sh = smem + (kt & 1) * STAGE;
    const int8_t* sl = sh + SA_BYTES;
    const int8_t* sb = sh + 2 * SA_BYTES;
    v4i xh[2][FM], xl[2][FM], w[2][FN];
    auto load = [&](int ks, int buf) {
      const int c = ks * 2 + khalf;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        xh[buf][i] = *reinterpret_cast<const v4i*>(sh + tile::lds_off<RB>(ra0 + i * 32, c));
        xl[buf][i] = *reinterpret_cast<const v4i*>(sl + tile::lds_off<RB>(ra0 + i * 32, c));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
        w[buf][j] = *reinterpret_cast<const v4i*>(sb + tile::lds_off<RB>(rb0 + j * 32, c)) & mask32;
    };
    load(0, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS) load(ks + 1, cur ^ 1);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          ah[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xh[cur][i], w[cur][j], ah[i][j], 0, 0, 0);
          al[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xl[cur][i], w[cur][j], al[i][j], 0, 0, 0);
        }
    }
  }

  // 32x32 output layout: lane l, register r holds row (r/4)*8 + (l/32)*4 + r%4, col l%32.
  const int row_w = m0 + wm * WTM, col_w = n0 + wn * WTN;
  auto combined = [&](int i, int j, int r) {
    return 128.0 * (double)ah[i][j][r] + (double)al[i][j][r];   // exact
  };
  if (ACC != nullptr) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gm = row_w + i * 32 + (r >> 2) * 8 + khalf * 4 + (r & 3);
          const int gn = col_w + j * 32 + (lane & 31);
          if (gm < M && gn < N) ACC[(size_t)gm * N + gn] = (long long)combined(i, j, r);
        }
  }
  if (Y != nullptr) {
    float sa_r[FM][16], sb_c[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = row_w + i * 32 + (r >> 2) * 8 + khalf * 4 + (r & 3);
        sa_r[i][r] = gm < M ? SA[gm] : 0.0f;
      }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int gn = col_w + j * 32 + (lane & 31);
      sb_c[j] = gn < N ? SB[gn] : 0.0f;
    }
    __syncthreads();   // every wave is done reading the last stage
    uint16_t* st = reinterpret_cast<uint16_t*>(smem) + wave * WTM * WTN;
    tile::store_tile32_bf16<WTM, WTN>(st, lane, Y, row_w, col_w, M, N, [&](int i, int j, int r) {
      return tile::bf16_rne(((float)combined(i, j, r) * sa_r[i][r]) * sb_c[j]);
    });
  }
}

struct HqCfg {
  int bm, bn, wm, wn;
  float rate;
};
// Eight or twelve waves (wave tiles 64 x 64, 32 x 96, 32 x 64): on MI355X the
// 12-wave 128 x 192 and 128 x 288 tiles beat every four- and eight-wave tile at
// the PixArt, SANA and CogVideoX shapes they are chosen for (PixArt MLP-down
// 67 -> 52 us, MLP-up 62 -> 51 us).  Rates: median per-tile rates of a
// graph-replayed sweep over nine shapes (chooser loss 0.6% on average).
// index, BM, BN, WM, WN, rate
#define TABIT_HQ_CONFIGS(X)     \
  X(0, 128, 256, 2, 4, 1.34f)   \
  X(1, 128, 288, 4, 3, 1.30f)   \
  X(2, 128, 192, 4, 3, 1.17f)   \
  X(3, 64, 64, 2, 2, 0.83f)
#define TABIT_HDESC(I, BM, BN, WM, WN, RATE) {BM, BN, WM, WN, RATE},
constexpr HqCfg kHqCfgs[] = {TABIT_HQ_CONFIGS(TABIT_HDESC)};
#undef TABIT_HDESC
constexpr int kNumHqCfgs = sizeof(kHqCfgs) / sizeof(kHqCfgs[0]);

template <int BM, int BN, int WM, int WN>
hipError_t launch_hq_cfg(const int8_t* xh, const int8_t* xl, const float* sa, const int8_t* wq,
                         const float* sw, int M, int N, int K, int kbits, uint16_t* y,
                         long long* acc, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const dim3 grid(tiles_m * tiles_n), block(WM * WN * 64);
  auto kern = gemm_hqdm_kernel<BM, BN, WM, WN>;
  if (ev0 != nullptr || ev1 != nullptr)
    hipExtLaunchKernelGGL(kern, grid, block, 0, s, ev0, ev1, 0, xh, xl, sa, wq, sw, M, N, K, kbits,
                          y, acc, tiles_m, tiles_n);
  else
    kern<<<grid, block, 0, s>>>(xh, xl, sa, wq, sw, M, N, K, kbits, y, acc, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

int hqdm_config_count() { return kNumHqCfgs; }

GemmConfig hqdm_config(int index) { return GemmConfig{kHqCfgs[index].bm, kHqCfgs[index].bn, 1}; }

// The busiest CU runs ceil(tiles / CUs) tiles; cost = that x BM x BN / rate.
int hqdm_config_choose(int M, int N, int K, int num_cus) {
  (void)K;
  if (num_cus <= 0) num_cus = 256;
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < kNumHqCfgs; ++i) {
    const HqCfg& c = kHqCfgs[i];
    const long long tiles = (long long)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const long long per_cu = (tiles + num_cus - 1) / num_cus;
    const double cost = (double)per_cu * c.bm * c.bn / c.rate;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = i;
    }
  }
  return best;
}

hipError_t launch_gemm_hqdm(int cfg, const int8_t* xh, const int8_t* xl, const float* sa,
                            const int8_t* wq, const float* sw, int M, int N, int K, int kbits,
                            uint16_t* y, long long* acc, hipStream_t stream, hipEvent_t ev0,
                            hipEvent_t ev1) {
#define TABIT_HCASE(I, BM, BN, WM, WN, RATE) \
  case I:                                   \
    return launch_hq_cfg<BM, BN, WM, WN>(xh, xl, sa, wq, sw, M, N, K, kbits, y, acc, stream, ev0, ev1);
  switch (cfg) {
    TABIT_HQ_CONFIGS(TABIT_HCASE)
    default: return hipErrorInvalidValue;
  }
#undef TABIT_HCASE
}

}  // namespace tabit
