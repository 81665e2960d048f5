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
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E2M1: lane l supplies
// 16 bytes = 32 consecutive K elements of row (l % 32) -- exactly one MX block
// -- and that block's E8M0 byte as its scale operand.  The tile skeleton is
// the INT8 GEMM's: packed operand stages of 128 bytes (256 elements) copied
// global->LDS by buffer loads into a double-buffered ring, one barrier per
// stage; each wave reads the next K-step's fragments and scale bytes from LDS
// while the matrix cores work on the current one.  The 8 scale bytes per row
// and stage go through registers (two words per row) into a small LDS table
// next to the data (their loads are issued before the stage's copies so
// waiting for them never waits for the copies).
#include "tabit_internal.h"
#include "tile_common.h"

namespace tabit {
namespace {

using tile::v4i;
using tile::v4u;
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int RB = 128;   // packed bytes per row per stage (256 elements)
constexpr int SPR = 8;    // scale bytes per row per stage

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM* WN * 64)
gemm_mxfp4_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ AE,
                  const uint8_t* __restrict__ B, const uint8_t* __restrict__ BE, int M, int N,
                  int K, float out_scale, uint16_t* __restrict__ Y, float* __restrict__ ACC,
                  int tiles_m, int tiles_n, const uint8_t* __restrict__ gate) {
  if (gate != nullptr && *gate != 1) return;   // device-selected format is not MXFP4
  constexpr int NT = WM * WN * 64, NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int KS = RB / 32;                     // 32-byte (64-element) K-steps per stage
  constexpr int DATA = (BM + BN) * RB;
  constexpr int SCL = (BM + BN) * SPR;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold whole 32x32 blocks");
  // the two stages, or the bf16 staging of the epilogue when that is larger
  constexpr int SMEM = 2 * DATA > BM * BN * 2 ? 2 * DATA : BM * BN * 2;
  __shared__ __attribute__((aligned(1024))) int8_t smem[SMEM];
  __shared__ __attribute__((aligned(16))) uint8_t sscale[2][SCL];

  int tm, tn;
  tile::tile_coords<4>(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int KB = K >> 1, KSB = K >> 5;            // packed bytes and scale bytes per row
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
  const auto rsa = tile::make_rsrc(A, (unsigned)M * (unsigned)KB);
  const auto rsb = tile::make_rsrc(B, (unsigned)N * (unsigned)KB);

  // Scale table of a stage: row r (0..BM-1 from AE, then BN rows from BE)
  // holds its 8 scale bytes; a thread moves whole rows, as two words when the
  // row's bytes are 4-byte aligned and all inside K (else byte by byte, 127 =
  // 2^0 past the end or past the last row).
  constexpr int RPT = (BM + BN + NT - 1) / NT;   // scale rows per thread
  static_assert(SPR == 8, "two words per row and stage");
  const bool words = (KSB & 3) == 0;
  uint32_t sreg[RPT][2];
  auto load_scales = [&](int kt) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = i * NT + tid;
      const uint8_t* src = nullptr;
      if (r < BM) {
        if (r < rows_a) src = AE + (size_t)(m0 + r) * KSB;
      } else if (r < BM + BN && r - BM < rows_b) {
        src = BE + (size_t)(n0 + r - BM) * KSB;
      }
      const int g0 = kt * SPR;
      uint32_t lo = 0x7F7F7F7Fu, hi = 0x7F7F7F7Fu;
      if (src != nullptr) {
        if (words && g0 + SPR <= KSB) {
          lo = *reinterpret_cast<const uint32_t*>(src + g0);
          hi = *reinterpret_cast<const uint32_t*>(src + g0 + 4);
        } else {
          lo = hi = 0u;
#pragma unroll
          for (int j = 0; j < SPR; ++j) {
            const uint32_t v = g0 + j < KSB ? src[g0 + j] : 127u;
            if (j < 4) lo |= v << (8 * j);
            else hi |= v << (8 * (j - 4));
          }
        }
      }
      sreg[i][0] = lo;
      sreg[i][1] = hi;
    }
  };
  auto store_scales = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = i * NT + tid;
      if (r < BM + BN)
        *reinterpret_cast<uint2*>(&sscale[buf][r * SPR]) = make_uint2(sreg[i][0], sreg[i][1]);
    }
  };
  auto issue = [&](int kt) {
    int8_t* dst = smem + (kt & 1) * DATA;
    tile::dma_stage<BM, NW, RB>(rsa, dst, m0, rows_a, KB, kt * RB, wave, lane);
    tile::dma_stage<BN, NW, RB>(rsb, dst + BM * RB, n0, rows_b, KB, kt * RB, wave, lane);
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

  const int ra0 = wm * WTM + (lane & 31), rb0 = wn * WTN + (lane & 31);
  const int khalf = lane >> 5;
  const int nk = (KB + RB - 1) / RB;

  load_scales(0);
  issue(0);
  store_scales(0);
  for (int kt = 0; kt < nk; ++kt) {
    tile::wait_vmcnt0();
    __syncthreads();
    const bool more = kt + 1 < nk;
    if (more) {
      load_scales(kt + 1);     // before the copies: waiting on these never waits on the copies
      issue(kt + 1);
    }
    const int8_t* sa = smem + (kt & 1) * DATA;
    const int8_t* sb = sa + BM * RB;
    const uint8_t* ssa = sscale[kt & 1];
    const uint8_t* ssb = ssa + BM * SPR;
    // fragments and scale bytes of K-step ks + 1 are read from LDS while the
    // matrix cores work on K-step ks
    v4i a[2][FM], b[2][FN];
    int ea[2][FM], eb[2][FN];
    auto load = [&](int ks, int buf) {
      const int c = ks * 2 + khalf;     // 16-byte chunk = one 32-element MX block
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = ra0 + i * 32;
        a[buf][i] = *reinterpret_cast<const v4i*>(sa + tile::lds_off<RB>(r, c));
        ea[buf][i] = ssa[r * SPR + c];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = rb0 + j * 32;
        b[buf][j] = *reinterpret_cast<const v4i*>(sb + tile::lds_off<RB>(r, c));
        eb[buf][j] = ssb[r * SPR + c];
      }
    };
    load(0, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS) load(ks + 1, cur ^ 1);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const v8i a8 = {a[cur][i][0], a[cur][i][1], a[cur][i][2], a[cur][i][3], 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v8i b8 = {b[cur][j][0], b[cur][j][1], b[cur][j][2], b[cur][j][3], 0, 0, 0, 0};
          // the weights as the first operand: lanes end with runs of four output columns
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, a8, acc[i][j], 4, 4, 0,
                                                                       eb[cur][j], 0, ea[cur][i]);
        }
      }
    }
    if (more) store_scales((kt + 1) & 1);
  }

  // Block (i, j) holds Y^T: lane l, register r is row i*32 + l%32 and column
  // j*32 + (r/4)*8 + (l/32)*4 + r%4 of the wave tile (four consecutive columns
  // per group of four registers), as in the INT8 GEMM's epilogue.
  const int row_w = m0 + wm * WTM, col_w = n0 + wn * WTN;
  if (ACC != nullptr) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int gm = row_w + i * 32 + (lane & 31);
          const int gn = col_w + j * 32 + g * 8 + khalf * 4;
          if (gm < M && gn < N)
            *reinterpret_cast<float4*>(ACC + (size_t)gm * N + gn) =
                make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                            acc[i][j][4 * g + 3]);
        }
  }
  if (Y != nullptr) {
    // bf16 pairs by the packed conversion; v_permlane32_swap pairs runs g and g + 1
    // so each lane holds 8 columns of its row, written to the wave's LDS staging as
    // 16 bytes; rows leave as full-line nontemporal stores
    constexpr int CH = WTN / 8, SW = CH & -CH;
    __syncthreads();  // every wave is done reading the last stage
    uint16_t* st = reinterpret_cast<uint16_t*>(smem) + wave * WTM * WTN;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        unsigned pk[4][2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const v2f lo = v2f{acc[i][j][4 * g] * out_scale, acc[i][j][4 * g + 1] * out_scale};
          const v2f hi = v2f{acc[i][j][4 * g + 2] * out_scale, acc[i][j][4 * g + 3] * out_scale};
          pk[g][0] = __builtin_bit_cast(unsigned, __builtin_convertvector(lo, v2bf));
          pk[g][1] = __builtin_bit_cast(unsigned, __builtin_convertvector(hi, v2bf));
        }
#pragma unroll
        for (int g = 0; g < 4; g += 2) {
          const auto s0 = __builtin_amdgcn_permlane32_swap(pk[g][0], pk[g + 1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(pk[g][1], pk[g + 1][1], false, false);
          const int lr = i * 32 + (lane & 31);
          const int ch = (j * 32 + (g + khalf) * 8) >> 3;
          *reinterpret_cast<v4u*>(st + lr * WTN + ((ch ^ (lr & (SW - 1))) << 3)) =
              v4u{s0[0], s1[0], s0[1], s1[1]};
        }
      }
    // the region is the wave's own: LDS operations of one wave complete in order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int it = 0; it < WTM * CH / 64; ++it) {
      const int idx = it * 64 + lane;
      const int lr = idx / CH, ch = idx % CH;
      const int gm = row_w + lr, gn = col_w + ch * 8;
      const v4u v = *reinterpret_cast<const v4u*>(st + lr * WTN + ((ch ^ (lr & (SW - 1))) << 3));
      if (gm < M && gn < N) __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(Y + (size_t)gm * N + gn));
    }
  }
}

struct CfgDesc {
  int bm, bn, wm, wn;
  float rate;   // relative throughput per CU on its tiles (fitted to MI355X sweeps)
};
// Eight waves of 32 x 64 or 64 x 64 on the large tiles (2-6% faster on the
// CogVideoX shapes than four waves of 64 x 64); 12- and 16-wave tiles with
// 256 rows spill here.  Rates: median per-tile rates of a graph-replayed sweep
// over seven DiT shapes.
// index, BM, BN, WM, WN, rate
#define TABIT_MX_CONFIGS(X)       \
  X(0, 128, 128, 4, 2, 1.00f)     \
  X(1, 256, 128, 4, 2, 1.02f)     \
  X(2, 128, 64, 2, 2, 0.84f)      \
  X(3, 64, 64, 2, 2, 0.69f)
#define TABIT_DESC(I, BM, BN, WM, WN, RATE) {BM, BN, WM, WN, RATE},
constexpr CfgDesc kCfgs[] = {TABIT_MX_CONFIGS(TABIT_DESC)};
#undef TABIT_DESC
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const uint8_t* xq, const uint8_t* xe, const uint8_t* wq, const uint8_t* we,
                      int M, int N, int K, float out_scale, uint16_t* y, float* acc,
                      hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, const uint8_t* gate) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const dim3 grid(tiles_m * tiles_n), block(WM * WN * 64);
  if (ev0 != nullptr || ev1 != nullptr)   // timestamps of this dispatch itself
    hipExtLaunchKernelGGL(gemm_mxfp4_kernel<BM, BN, WM, WN>, grid, block, 0, s, ev0, ev1, 0, xq, xe,
                          wq, we, M, N, K, out_scale, y, acc, tiles_m, tiles_n, gate);
  else
    gemm_mxfp4_kernel<BM, BN, WM, WN><<<grid, block, 0, s>>>(xq, xe, wq, we, M, N, K, out_scale, y,
                                                             acc, tiles_m, tiles_n, gate);
  return hipGetLastError();
}

}  // namespace

int mx_config_count() { return kNumCfgs; }

GemmConfig mx_config(int index) { return GemmConfig{kCfgs[index].bm, kCfgs[index].bn, 1}; }

// Same model as the INT8 GEMM's: the busiest CU runs ceil(tiles / CUs) tiles;
// cost = that x BM x BN / rate, rates fitted to sweeps of every configuration
// over the 4-bit layers' shapes on MI355X.
int mx_config_choose(int M, int N, int K, int num_cus) {
  (void)K;
  if (num_cus <= 0) num_cus = 256;
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < kNumCfgs; ++i) {
    const CfgDesc& c = kCfgs[i];
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

hipError_t launch_gemm_mxfp4(int cfg, const uint8_t* xq, const uint8_t* xe, const uint8_t* wq,
                             const uint8_t* we, int M, int N, int K, float out_scale, uint16_t* y,
                             float* acc, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1,
                             const uint8_t* gate) {
#define TABIT_CASE(I, BM, BN, WM, WN, RATE) \
  case I:                                           \
    return launch_cfg<BM, BN, WM, WN>(xq, xe, wq, we, M, N, K, out_scale, y, acc, stream, \
                                      ev0, ev1, gate);
  switch (cfg) {
    TABIT_MX_CONFIGS(TABIT_CASE)
    default: return hipErrorInvalidValue;
  }
#undef TABIT_CASE
}

}  // namespace tabit
