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
// 16 bytes = 32 K elements of row (l % 32) -- exactly one MX block -- and a
// scale word whose byte opsel is that block's E8M0 scale.  Operands move
// global->LDS in stages of 128 packed bytes (256 elements) per row by buffer
// loads straight into LDS, through a ring of two or three stages with the
// next one or two in flight while the matrix cores work on the current one;
// a stage's 8 scale bytes per row come along as a small table in LDS (4-byte
// copies, when K is a multiple of 128) or, otherwise, as per-lane byte loads
// into registers.  Each wave reads the next K-step's fragments from LDS while
// the matrix cores work on the current one.
//
// What keeps the copies in flight: one LDS array (with several, the compiler
// orders every read of an array after all copies into it still in flight), a
// barrier that waits only for LDS traffic (the copies a stage needs are waited
// for explicitly, by count), and every iteration issuing its stage, also past
// the end of K, so the count is the same on every path.
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

// E2M1 x E2M1 block-scaled MFMA; byte sel (0..3) of each scale word is the
// scale of the lane's block (sel is a constant once the K-step loop unrolls)
__device__ __forceinline__ v16f mfma_fp4(int sel, v8i a, v8i b, v16f c, int sa, int sb) {
  switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 1, sa, 1, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 2, sa, 2, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 3, sa, 3, sb);
  }
}

// One 4-byte copy of a stage's scale table: 32 rows (two lanes per row) of
// operand rows row0 + r, bytes g .. g + 3 of each (g < row length or nothing).
__device__ __forceinline__ void copy_scale_rows(__amdgpu_buffer_rsrc_t rs, int8_t* dst, int r,
                                                int rows_valid, int row0, int ksb, int g) {
  const unsigned off = r < rows_valid && g < ksb ? (unsigned)(row0 + r) * ksb + g : tile::kOOB;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (tile::lds_ptr_t)dst, 4, off, 0, 0, 0);
}

template <int BM, int BN, int WM, int WN, int NST, bool SW4>
__global__ void __launch_bounds__(WM* WN * 64)
gemm_mxfp4_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ AE,
                  const uint8_t* __restrict__ B, const uint8_t* __restrict__ BE, int M, int N,
                  int K, float out_scale, uint16_t* __restrict__ Y, float* __restrict__ ACC,
                  int tiles_m, int tiles_n, const uint8_t* __restrict__ gate) {
  if (gate != nullptr && *gate != 1) return;   // device-selected format is not MXFP4
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int KS = RB / 32;                     // 32-byte (64-element) K-steps per stage
  constexpr int DATA = (BM + BN) * RB;
  constexpr int DPW = DATA / 1024 / NW;           // copies per wave per stage
  // a stage's scale table: BM + BN rows of 8 bytes (the stage's 32-element
  // blocks), copied 32 rows per instruction (whole instructions per wave, the
  // last ones past the table reading out of range into padding); without
  // 4-byte aligned scale words each lane loads its rows' bytes into registers
  constexpr int SIN = (BM + BN) / 32;
  constexpr int SCW = SW4 ? (SIN + NW - 1) / NW : 0;
  constexpr int SCL = SCW * NW * 256;             // LDS bytes of a stage's scale table
  constexpr int SPW = SW4 ? SCW : (FM + FN) * 4;  // scale loads per wave per stage
  constexpr int PER_STAGE = DPW + SPW;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold whole 32x32 blocks");
  static_assert(NST == 2 || NST == 3, "two or three LDS stages");
  static_assert(NST == 2 || (BM % (8 * NW) == 0 && BN % (8 * NW) == 0),
                "the three-stage waits count loads per wave: every wave copies the same share");
  static_assert((NST - 1) * PER_STAGE < 64, "vmcnt range");
  // the stages (or the bf16 staging of the epilogue when that is larger), then
  // the stages' scale tables
  constexpr int SMEM = NST * DATA > BM * BN * 2 ? NST * DATA : BM * BN * 2;
  static_assert(SMEM + NST * SCL <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) int8_t smem[SMEM + NST * SCL];

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
  const auto rsae = tile::make_rsrc(AE, (unsigned)M * (unsigned)KSB);
  const auto rsbe = tile::make_rsrc(BE, (unsigned)N * (unsigned)KSB);

  // Lane l reads rows ra0 + 32 i of A and rb0 + 32 j of B.  At K-step ks of a
  // stage the lanes of half h = l / 32 take 16-byte chunk 4 h + ks (32 FP4
  // values, one MX block), the same chunk for both operands, so a lane's four
  // block scales of a stage are the 4 consecutive scale bytes 4 h .. 4 h + 3 of
  // the stage's 8; byte ks of that word is the MFMA's scale at K-step ks.
  const int ra0 = wm * WTM + (lane & 31), rb0 = wn * WTN + (lane & 31);
  const int khalf = lane >> 5;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "rows ra0 + 32 i and rb0 + 32 j share a swizzle");
  const int sw = tile::swz<RB>(ra0);
  const int nk = (KB + RB - 1) / RB;

  // scale-word offsets of the lane's rows (past M or N: out of range, reads 0)
  unsigned eoff[FM + FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
    eoff[i] = ra0 + i * 32 < rows_a ? (unsigned)(m0 + ra0 + i * 32) * KSB + khalf * 4 : tile::kOOB;
#pragma unroll
  for (int j = 0; j < FN; ++j)
    eoff[FM + j] = rb0 + j * 32 < rows_b ? (unsigned)(n0 + rb0 + j * 32) * KSB + khalf * 4
                                         : tile::kOOB;
  // Scale bytes past the row's end read as 0 (E8M0 2^-127; their FP4 values are
  // zeros).  With K a multiple of 128 a lane's word lies wholly inside or
  // outside the row and is one load; otherwise it comes as 4 byte loads, kept
  // apart until the stage is used (assembling them at once would wait for them).
  typedef int Scales[FM + FN][SW4 ? 1 : 4];
  auto load_scales = [&](int kt, Scales& e) {
    const int g = kt * SPR + khalf * 4;
#pragma unroll
    for (int r = 0; r < FM + FN; ++r) {
      const auto rs = r < FM ? rsae : rsbe;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        e[r][q] = __builtin_amdgcn_raw_buffer_load_b8(rs, g + q < KSB ? eoff[r] + kt * SPR + q : tile::kOOB,
                                                      0, 0);
    }
  };
  auto scale_word = [&](const Scales& e, int r) {
    return e[r][0] | (e[r][1] << 8) | (e[r][2] << 16) | (e[r][3] << 24);
  };
  // 4-byte copies into the stage's table: lane L of copy j moves bytes
  // 4 (L % 2) .. 4 (L % 2) + 3 of row 32 j + L / 2 (rows of A, then of B)
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto copy_scales = [&](int kt, int buf) {
    const int g = kt * SPR + (lane & 1) * 4;
#pragma unroll
    for (int q = 0; q < SCW; ++q) {
      const int j = q * NW + wave_u;   // wave-uniform
      int8_t* dst = smem + SMEM + buf * SCL + j * 256;
      if (j * 32 < BM)
        copy_scale_rows(rsae, dst, j * 32 + (lane >> 1), rows_a, m0, KSB, g);
      else   // rows past BN in the padding copies
        copy_scale_rows(rsbe, dst, j * 32 - BM + (lane >> 1), rows_b, n0, KSB, g);
    }
  };
  // A stage's loads: its scale words, then its copies into LDS buffer buf.  The
  // waits below count on every load of a stage being issued before any load
  // of the next (vmcnt retires loads in issue order); the compiler fences keep
  // that order.
  auto issue = [&](int kt, int buf, Scales& e) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if constexpr (SW4) copy_scales(kt, buf);
    else load_scales(kt, e);
    int8_t* dst = smem + buf * DATA;
    tile::dma_stage<BM, NW, RB>(rsa, dst, m0, rows_a, KB, kt * RB, wave, lane);
    tile::dma_stage<BN, NW, RB>(rsb, dst + BM * RB, n0, rows_b, KB, kt * RB, wave, lane);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

  // Stage t's scales in registers e[t % NST], its data in LDS buffer t % NST.
  // Every iteration issues the stage NST-1 ahead, also past the last one
  // (out-of-range loads return zeros into a buffer no one reads), so every
  // path carries the same loads in flight: at the top of iteration kt only
  // the NST-2 stages after kt may still be pending.
  Scales e[NST];
#pragma unroll
  for (int t = 0; t < NST - 1; ++t) issue(t, t, e[t]);
  for (int k0 = 0; k0 < nk; k0 += NST) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int kt = k0 + s;
      if (kt >= nk) break;   // uniform
      tile::wait_vmcnt<(NST - 2) * PER_STAGE>();
      tile::lds_barrier();   // stage kt visible to all; the buffer of stage kt-1 free
      issue(kt + NST - 1, (s + NST - 1) % NST, e[(s + NST - 1) % NST]);
      int ew[FM + FN];
      if constexpr (SW4) {
        const int8_t* ss = smem + SMEM + s * SCL + khalf * 4;
#pragma unroll
        for (int i = 0; i < FM; ++i) ew[i] = *reinterpret_cast<const int*>(ss + (ra0 + i * 32) * SPR);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          ew[FM + j] = *reinterpret_cast<const int*>(ss + (BM + rb0 + j * 32) * SPR);
      } else {
#pragma unroll
        for (int r = 0; r < FM + FN; ++r) ew[r] = scale_word(e[s], r);
      }
      const int8_t* sa = smem + s * DATA + ra0 * RB;
      const int8_t* sb = smem + s * DATA + BM * RB + rb0 * RB;
      // fragments of K-step ks + 1 are read from LDS while the matrix cores
      // work on K-step ks; rows ra0 + 32 i and rb0 + 32 j share one swizzle,
      // so a K-step's chunk offset is one value for both operands
      v4i a[2][FM], b[2][FN];
      auto load = [&](int ks, int buf) {
        const int co = ((khalf * 4 + ks) ^ sw) << 4;
#pragma unroll
        for (int i = 0; i < FM; ++i) a[buf][i] = *reinterpret_cast<const v4i*>(sa + i * 32 * RB + co);
#pragma unroll
        for (int j = 0; j < FN; ++j) b[buf][j] = *reinterpret_cast<const v4i*>(sb + j * 32 * RB + co);
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
            // the weights as the first operand: lanes end with runs of four
            // output columns
            acc[i][j] = mfma_fp4(ks, b8, a8, acc[i][j], ew[FM + j], ew[i]);
          }
        }
      }
    }
  }

  // the stages issued past K may still be landing (zeros) in LDS: drain them
  // before the workgroup ends or anything below reuses LDS
  tile::wait_vmcnt0();

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
  int bm, bn, wm, wn, nst;
  float rate;     // relative throughput per CU on its tiles (fitted to MI355X sweeps)
  int k128;       // only for K a multiple of 128 (its byte-scale variant spills)
};
// The 256 x 256 tile: sixteen waves of 64 x 64, two stages (136 KB of LDS);
// 256 x 192: twelve waves of 64 x 64, two stages (124 KB); 256 x 128: eight
// waves of 64 x 64, three stages (156 KB); the others eight or four waves, two
// stages.  Rates: per-CU tile rates measured on the CogVideoX MLP-up, MLP-down,
// QKV and out linears (17776 x {7680, 1920, 5760, 1920} x {1920, 7680, 1920,
// 1920}), PixArt's MLP-up (4096 x 4608 x 1152) and 8192^3: 256 x 256 runs
// 1.30-1.56x the 128 x 128 tile's rate per CU, 256 x 128 0.97-1.21x; 256 x 192
// is the pick where N = 1920 leaves the 256-wide tiles a mostly empty last
// round (CogVideoX MLP-down 176 -> 158 us, out 59 -> 53 us).
// index, BM, BN, WM, WN, LDS stages, rate, K multiple of 128 only
#define TABIT_MX_CONFIGS(X)             \
  X(0, 128, 128, 4, 2, 2, 1.00f, 0)     \
  X(1, 256, 128, 4, 2, 3, 1.12f, 0)     \
  X(2, 128, 64, 2, 2, 2, 0.84f, 0)      \
  X(3, 64, 64, 2, 2, 2, 0.69f, 0)       \
  X(4, 256, 256, 4, 4, 2, 1.40f, 1)     \
  X(5, 256, 192, 4, 3, 2, 1.20f, 0)
#define TABIT_DESC(I, BM, BN, WM, WN, NST, RATE, K128) {BM, BN, WM, WN, NST, RATE, K128},
constexpr CfgDesc kCfgs[] = {TABIT_MX_CONFIGS(TABIT_DESC)};
#undef TABIT_DESC
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

template <int BM, int BN, int WM, int WN, int NST>
hipError_t launch_cfg(const uint8_t* xq, const uint8_t* xe, const uint8_t* wq, const uint8_t* we,
                      int M, int N, int K, float out_scale, uint16_t* y, float* acc,
                      hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, const uint8_t* gate) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const dim3 grid(tiles_m * tiles_n), block(WM * WN * 64);
  // a stage's scale words are 4-byte aligned when K is a multiple of 128
  auto kern = K % 128 == 0 ? gemm_mxfp4_kernel<BM, BN, WM, WN, NST, true>
                           : gemm_mxfp4_kernel<BM, BN, WM, WN, NST, false>;
  if (ev0 != nullptr || ev1 != nullptr)   // timestamps of this dispatch itself
    hipExtLaunchKernelGGL(kern, grid, block, 0, s, ev0, ev1, 0, xq, xe, wq, we, M, N, K, out_scale,
                          y, acc, tiles_m, tiles_n, gate);
  else
    kern<<<grid, block, 0, s>>>(xq, xe, wq, we, M, N, K, out_scale, y, acc, tiles_m, tiles_n, gate);
  return hipGetLastError();
}

}  // namespace

int mx_config_count() { return kNumCfgs; }

GemmConfig mx_config(int index) { return GemmConfig{kCfgs[index].bm, kCfgs[index].bn, 1}; }

// Same model as the INT8 GEMM's: the busiest CU runs ceil(tiles / CUs) tiles;
// cost = that x BM x BN / rate, rates fitted to sweeps of every configuration
// over the 4-bit layers' shapes on MI355X.  Tiles marked for K a multiple of
// 128 are left out for other K.
int mx_config_choose(int M, int N, int K, int num_cus) {
  if (num_cus <= 0) num_cus = 256;
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < kNumCfgs; ++i) {
    const CfgDesc& c = kCfgs[i];
    if (c.k128 && K % 128 != 0) continue;
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
#define TABIT_CASE(I, BM, BN, WM, WN, NST, RATE, K128) \
  case I:                                                \
    return launch_cfg<BM, BN, WM, WN, NST>(xq, xe, wq, we, M, N, K, out_scale, y, acc, stream, \
                                           ev0, ev1, gate);
  switch (cfg) {
    TABIT_MX_CONFIGS(TABIT_CASE)
    default: return hipErrorInvalidValue;
  }
#undef TABIT_CASE
}

}  // namespace tabit
