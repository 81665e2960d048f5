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
// fragment is loaded once per K-step and reused against each retained plane,
// the analogue of the Temporal-Precision Engine keeping activation planes on
// chip and streaming only the selected weight planes.  A plane is the byte
// W & (1 << b) read as int8 ({0, 2^b}, or {0, -128} for b = 7), so its MFMA
// product is exactly c_b (Xq . W_b^T).
//
// Both operands are K-contiguous ([M][K] and [N][K]).  A workgroup of WM x WN
// waves computes a BM x BN tile; K advances in 128-byte stages copied straight
// from global memory by buffer loads (no register staging; rows and chunks out
// of range arrive as zeros) into an NST-deep ring of LDS stages: up to NST-1
// stages are in flight, so the copy latency (an L2 miss costs about as much as
// a stage of MFMAs) hides under the compute.  One barrier per stage; it waits
// only for LDS accesses, each wave having first waited by count for its own
// copies of the stage.  The step's LSB mask is applied to the weight
// fragments as they come out of LDS (four v_and per 16-byte fragment).  The
// matrix-core op is v_mfma_i32_32x32x32_i8 (it sustains ~90% of the chip's INT8
// rate with a few independent accumulators per wave), with the weight fragment
// as its first operand so that every lane ends with runs of four consecutive
// output columns.  The epilogue scales in fp32 (the tile's scales were copied
// into LDS at the start), rounds pairs to bf16 with the packed conversion,
// writes each pair of runs to its wave's LDS staging as 16 bytes, from where
// rows go out as full-line nontemporal stores.
//
// K split inside the workgroup (KW > 1), for shapes whose tiles fit in one
// round over the CUs (a few tokens, or a long K): KW groups of WM x WN waves
// each walk a contiguous range
// of the K stages through their own LDS ring; groups 1..KW-1 then hand their
// int32 accumulators to group 0 through LDS (integer sums: the result equals
// the unsplit one bit for bit) and group 0 runs the epilogue.  Every wave
// takes part in every barrier.
#include "tabit_internal.h"
#include "tile_common.h"

namespace tabit {
namespace {

using tile::v4i;
using tile::v4u;
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

template <int BM, int BN, int WM, int WN, int RB, int NST, int KW, bool BITSERIAL>
__global__ void __launch_bounds__(WM* WN * KW * 64)
gemm_i8_kernel(const int8_t* __restrict__ A, const float* __restrict__ SA,
               const int8_t* __restrict__ B, const float* __restrict__ SB, int M, int N, int K,
               int kbits, uint16_t* __restrict__ Y, int32_t* __restrict__ ACC, int tiles_m,
               int tiles_n, const uint8_t* __restrict__ gate) {
  if (gate != nullptr && *gate != 0) return;   // device-selected format is not INT8
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;   // 32 x 32 MFMA blocks per wave
  constexpr int KS = RB / 32;                   // MFMA K-steps (32 bytes) per stage
  constexpr int STAGE = (BM + BN) * RB;
  constexpr int DPW = STAGE / 1024 / NW;        // DMA instructions per wave per stage (at least)
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold whole 32x32 blocks");
  static_assert(NST >= 2 && NST <= 4, "2 to 4 LDS stages");
  static_assert(KW >= 1 && (KW - 1) * BM * BN * 4 <= KW * NST * STAGE,
                "the K groups' partial accumulators must fit in the LDS stages");
  static_assert(NW * KW * 64 <= 1024, "at most 1024 threads per workgroup");
  // Deeper rings wait by count: DPW is the smallest per-wave share of a
  // stage's copies; a wave that copies one block more (blocks that do not
  // split evenly) then also waits for one copy of the next stage, which is
  // only stricter.
  // the ring (the K groups' partial sums and the epilogue's bf16 staging reuse it,
  // the staging extending it where larger), then the tile's scales when they fit:
  // SA of its BM rows, SB of its BN columns (padded to whole waves of 64 entries)
  constexpr int RING = KW * NST * STAGE;
  constexpr int BASE = RING > BM * BN * 2 ? RING : BM * BN * 2;
  constexpr int NSCALE = BM + (BN + 63) / 64 * 64;
  constexpr bool SCALES_IN_LDS = BASE + NSCALE * 4 <= 160 * 1024;
  static_assert(BM % 64 == 0 && NSCALE / 64 <= NW * KW, "one scale wave per 64 entries");
  __shared__ __attribute__((aligned(1024))) int8_t smem[BASE + (SCALES_IN_LDS ? NSCALE * 4 : 0)];
  float* s_scale = reinterpret_cast<float*>(smem + BASE);

  int tm, tn;
  tile::tile_coords<4>(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  // K group and wave within it (compile-time 0 and the wave id without a split)
  const int group = KW > 1 ? (tid >> 6) / NW : 0;
  const int wave = KW > 1 ? (tid >> 6) % NW : (tid >> 6), lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  int8_t* ring = smem + group * NST * STAGE;
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
  const auto rsa = tile::make_rsrc(A, (unsigned)M * (unsigned)K);
  const auto rsb = tile::make_rsrc(B, (unsigned)N * (unsigned)K);

  if constexpr (SCALES_IN_LDS) {
    // the epilogue's scales, copied once by 4-byte buffer loads straight into LDS
    // (rows and columns past M and N read as 0); the first stage's wait covers them
    const int w_all = tid >> 6;
    if (w_all < NSCALE / 64) {
      const int t = w_all * 64 + lane;
      if (t < BM) {   // BM is a multiple of 64: the wave's entries are all rows
        const auto rs = tile::make_rsrc(SA, (unsigned)M * 4u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (tile::lds_ptr_t)(s_scale + w_all * 64), 4,
                                                 (unsigned)(m0 + t) * 4u, 0, 0, 0);
      } else {
        const auto rs = tile::make_rsrc(SB, (unsigned)N * 4u);
        const unsigned off = t - BM < BN ? (unsigned)(n0 + t - BM) * 4u : tile::kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (tile::lds_ptr_t)(s_scale + w_all * 64), 4,
                                                 off, 0, 0, 0);
      }
    }
  }

  const uint32_t m8 = (0xFFu << kbits) & 0xFFu;
  const int mask32 = (int)(m8 * 0x01010101u);

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16i{};

  // operand rows this lane reads: A rows wm*WTM + i*32 + lane%32, B likewise
  const int ra0 = wm * WTM + (lane & 31), rb0 = wn * WTN + (lane & 31);
  const int khalf = lane >> 5;   // which 16-byte half of the 32-byte K-step

  // this group's stages [kt0, kt0 + nk); every group runs `trips` iterations
  const int S = (K + RB - 1) / RB;
  const int trips = KW > 1 ? (S + KW - 1) / KW : S;
  const int kt0 = KW > 1 ? group * trips : 0;
  const int nk = KW > 1 ? max(0, min(S - kt0, trips)) : S;
  auto issue = [&](int it) {
    int8_t* dst = ring + (it % NST) * STAGE;
    const int kb = (kt0 + it) * RB;
    tile::dma_stage<BM, NW, RB>(rsa, dst, m0, rows_a, K, kb, wave, lane);
    tile::dma_stage<BN, NW, RB>(rsb, dst + BM * RB, n0, rows_b, K, kb, wave, lane);
  };
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nk) issue(s);
  for (int kt = 0; kt < trips; ++kt) {
    // stage kt has landed once at most (stages issued after it) x DPW copies are pending
    const int ahead = min(NST - 2, nk - 1 - kt);
    if (NST >= 4 && ahead >= 2) tile::wait_vmcnt<(NST >= 4 ? 2 : 0) * DPW>();
    else if (NST >= 3 && ahead >= 1) tile::wait_vmcnt<(NST >= 3 ? 1 : 0) * DPW>();
    else tile::wait_vmcnt<0>();
    // stage kt visible to all; stage kt-1's buffer free for reuse (the copies
    // of later stages stay in flight: __syncthreads would wait for them too)
    tile::lds_barrier();
    if constexpr (KW > 1) {
      if (kt >= nk) continue;   // this group's range is done (the barrier above still counts it)
    }
    if (kt + NST - 1 < nk) issue(kt + NST - 1);
    const int8_t* sa = ring + (kt % NST) * STAGE;
    const int8_t* sb = sa + BM * RB;
    v4i a[2][FM], b[2][FN];
    auto load = [&](int ks, int buf) {
      const int c = ks * 2 + khalf;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[buf][i] = *reinterpret_cast<const v4i*>(sa + tile::lds_off<RB>(ra0 + i * 32, c));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[buf][j] = *reinterpret_cast<const v4i*>(sb + tile::lds_off<RB>(rb0 + j * 32, c));
    };
    load(0, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS) load(ks + 1, cur ^ 1);
      if constexpr (!BITSERIAL) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v4i bm = b[cur][j] & mask32;   // TASQ LSB mask on the staged weight tile
#pragma unroll
          for (int i = 0; i < FM; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bm, a[cur][i], acc[i][j], 0, 0, 0);
        }
      } else {
        for (int p = 7; p >= kbits; --p) {
          const int pm = (int)(0x01010101u << p);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const v4i bp = b[cur][j] & pm;
#pragma unroll
            for (int i = 0; i < FM; ++i)
              acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bp, a[cur][i], acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  }

  // the epilogue's scales when they are not in LDS: loaded here, so that their
  // latency overlaps the K groups' exchange below
  const int row_w = m0 + wm * WTM, col_w = n0 + wn * WTN;
  float sa_i[FM];
  float4 sw_g[FN][4];
  if (Y != nullptr && (KW == 1 || group == 0)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int t = wm * WTM + i * 32 + (lane & 31);
      if constexpr (SCALES_IN_LDS) sa_i[i] = s_scale[t];
      else sa_i[i] = m0 + t < M ? SA[m0 + t] : 0.0f;
    }
    const bool sb16 = (reinterpret_cast<uintptr_t>(SB) & 15) == 0;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gn = n0 + wn * WTN + j * 32 + g * 8 + khalf * 4;   // first column of the half-run
        if constexpr (SCALES_IN_LDS) {
          sw_g[j][g] = float4{};        // read from LDS where used
        } else if (sb16 && gn + 3 < N) {
          sw_g[j][g] = *reinterpret_cast<const float4*>(SB + gn);
        } else {
          sw_g[j][g] = make_float4(gn < N ? SB[gn] : 0.0f, gn + 1 < N ? SB[gn + 1] : 0.0f,
                                   gn + 2 < N ? SB[gn + 2] : 0.0f, gn + 3 < N ? SB[gn + 3] : 0.0f);
        }
      }
  }

  if constexpr (KW > 1) {
    // groups 1..KW-1 hand their partial sums to group 0: v4i q of lane t of
    // wave w in group g at part[((g - 1) * NQ + q) * NW * 64 + w * 64 + t]
    constexpr int NQ = FM * FN * 4, GT = NW * 64;
    v4i* part = reinterpret_cast<v4i*>(smem);
    const int t = wave * 64 + lane;
    __syncthreads();   // every group is done reading its ring
    if (group > 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            part[((group - 1) * NQ + (i * FN + j) * 4 + g4) * GT + t] =
                v4i{acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                    acc[i][j][4 * g4 + 3]};
    }
    __syncthreads();
    if (group == 0) {
      for (int g = 1; g < KW; ++g)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const v4i v = part[((g - 1) * NQ + (i * FN + j) * 4 + g4) * GT + t];
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][j][4 * g4 + e] += v[e];
            }
    }
  }
  const bool out = KW == 1 || group == 0;   // the waves that hold the tile's sums

  // ------------------------------------------------------------ epilogue
  // The weights are the MFMA's first operand, so block (i, j) holds Y^T: lane l,
  // register r is output row m = i*32 + l%32 and column n = j*32 + (r/4)*8 +
  // (l/32)*4 + r%4 of the wave tile -- four consecutive columns per group g = r/4
  // of four registers; lanes l and l + 32 hold the two halves of an 8-column run.
  // int32 results go out as 16 bytes per run.  bf16 results: each run is packed
  // to two words, then one v_permlane32_swap per word pairs runs g and g + 1, so
  // lane l holds run g's 8 columns and lane l + 32 run g + 1's, written to the
  // LDS staging as 16 bytes (8 writes per lane for a 64 x 64 wave tile instead
  // of 64 two-byte ones).
  if (ACC != nullptr && out) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int gm = row_w + i * 32 + (lane & 31);
          const int gn = col_w + j * 32 + g * 8 + khalf * 4;
          if (gm < M && gn < N)
            *reinterpret_cast<v4i*>(ACC + (size_t)gm * N + gn) =
                v4i{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        }
  }
  if (Y != nullptr) {
    // stage the wave's bf16 tile in LDS (its own WTM x WTN region over the ring:
    // every wave must be done reading the last stage or the partial sums first),
    // one 16-byte write per run pair, then read it back row by row for full-line
    // nontemporal stores (128 contiguous bytes per row per 64 columns: partial-line
    // or write-allocating stores measured up to 3x and 1.3x slower)
    constexpr int CH = WTN / 8, SW = CH & -CH;   // 16-byte chunks per staged row; swizzle span
    __syncthreads();
    if (!out) return;                            // K groups 1.. hold no output
    uint16_t* st = reinterpret_cast<uint16_t*>(smem) + wave * WTM * WTN;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      v2u pk[FM][4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 sw =
            SCALES_IN_LDS ? *reinterpret_cast<const float4*>(s_scale + BM + wn * WTN + j * 32 + g * 8 +
                                                              khalf * 4)
                          : sw_g[j][g];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          // y = bf16_rne(((float)acc * sa) * sw): two fp32 multiplies in this order,
          // then the packed round-to-nearest-even conversion
          const v2f lo = v2f{((float)acc[i][j][4 * g] * sa_i[i]) * sw.x,
                             ((float)acc[i][j][4 * g + 1] * sa_i[i]) * sw.y};
          const v2f hi = v2f{((float)acc[i][j][4 * g + 2] * sa_i[i]) * sw.z,
                             ((float)acc[i][j][4 * g + 3] * sa_i[i]) * sw.w};
          pk[i][g] = v2u{__builtin_bit_cast(unsigned, __builtin_convertvector(lo, v2bf)),
                         __builtin_bit_cast(unsigned, __builtin_convertvector(hi, v2bf))};
        }
      }
#pragma unroll
      for (int g = 0; g < 4; g += 2)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          // lanes 32-63 of run g's words trade places with lanes 0-31 of run g + 1's:
          // lane l then holds the 8 columns of run g + l / 32 of its row
          const auto s0 = __builtin_amdgcn_permlane32_swap(pk[i][g][0], pk[i][g + 1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(pk[i][g][1], pk[i][g + 1][1], false, false);
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
  int bm, bn, wm, wn, rb, nst, kw;
  float rate;       // relative throughput per CU on its tiles (fitted to MI355X sweeps)
  int min_stages;   // K-split and deeper-ring variants: taken only from this many K stages on
};
// Twelve or sixteen waves per large tile (wave tiles of 64 x 64 or 64 x 96):
// on MI355X these beat the same tiles with eight waves of 128 x 64 by 3-15%
// at every DiT shape (more waves per SIMD keep the matrix cores fed between
// barriers), and the 288- and 192-wide tiles split N = 1152, 1920, 4608, 7680
// into whole rounds of tiles over the CUs.  Rates are the median per-tile
// rates of a graph-replayed sweep of every tile over 22 DiT shapes (the
// chooser then loses 1.1% on average, at most 6%, to the best tile).
// The 64 x 64 tile splits K over three or four groups of 2 x 2 waves, whichever
// walks fewer stages per group (then fewer groups): four groups take
// 64 x 1152 x 4608 from 13.4 to 12.4 us and 16 x 2240 x 5600 from 21.7 to
// 20.5 us; at K = 1152 both walk three stages and three groups are faster.
// The K-split 128 x 192 and 128 x 96 tiles (two groups of six waves, each
// with its own ring) pay only on long K: PixArt MLP-down 4096 x 1152 x 4608
// 31.8 -> 29.3 us, 4096 x 1280 x 5120 35.7 -> 33.9 us, SANA MLP-down
// 1024 x 2240 x 5600 42.7 -> 38.9 us, but 11.8 -> 12.8 us at K = 1152.
// The three-stage 128 x 192 and 128 x 96 tiles keep two stages in flight
// instead of one; they replace the two-stage tile from 16 K stages on (below
// the K split's 32): SANA MLP-up 1024 x 5600 x 2240 24.5-25.1 -> 21.6-21.9 us,
// SANA out 1024 x 2240 x 2240 (128 x 96) 13.7 -> 12.8-13.0 us; at 9-10 stages
// (4096 x 1152 x 1152, 4096 x 1280 x 1280) they are 3-5% slower, and a
// three-stage 128 x 128 tile was 11% slower at 1024 x 6720 x 2240.
// index, BM, BN, WM, WN, stage row bytes, LDS stages, K groups, rate, min stages
#define TABIT_I8_CONFIGS(X)                    \
  X(0, 256, 256, 4, 4, 128, 2, 1, 1.00f, 0)     \
  X(1, 256, 288, 4, 3, 128, 2, 1, 1.04f, 0)     \
  X(2, 256, 192, 4, 3, 128, 2, 1, 0.88f, 0)     \
  X(3, 128, 128, 4, 2, 128, 2, 1, 0.65f, 0)     \
  X(4, 128, 96, 4, 3, 128, 2, 1, 0.58f, 0)      \
  X(5, 64, 64, 2, 2, 128, 2, 1, 0.48f, 0)       \
  X(6, 128, 192, 4, 3, 128, 2, 1, 0.71f, 0)     \
  X(7, 64, 64, 2, 2, 128, 2, 3, 0.48f, 2)       \
  X(8, 128, 192, 2, 3, 128, 2, 2, 0.71f, 32)   \
  X(9, 128, 96, 2, 3, 128, 2, 2, 0.58f, 32)    \
  X(10, 64, 64, 2, 2, 128, 2, 4, 0.48f, 2)      \
  X(11, 128, 192, 4, 3, 128, 3, 1, 0.71f, 16)   \
  X(12, 128, 96, 4, 3, 128, 3, 1, 0.58f, 16)
#define TABIT_DESC(I, BM, BN, WM, WN, RB, NST, KW, RATE, MS) {BM, BN, WM, WN, RB, NST, KW, RATE, MS},
constexpr CfgDesc kCfgs[] = {TABIT_I8_CONFIGS(TABIT_DESC)};
#undef TABIT_DESC
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

template <int BM, int BN, int WM, int WN, int RB, int NST, int KW>
hipError_t launch_cfg(bool bitserial, const int8_t* xq, const float* sa, const int8_t* wq,
                      const float* sw, int M, int N, int K, int kbits, uint16_t* y, int32_t* acc,
                      hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, const uint8_t* gate) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const dim3 grid(tiles_m * tiles_n), block(WM * WN * KW * 64);
  auto kern = bitserial ? gemm_i8_kernel<BM, BN, WM, WN, RB, NST, KW, true>
                        : gemm_i8_kernel<BM, BN, WM, WN, RB, NST, KW, false>;
  if (ev0 != nullptr || ev1 != nullptr)   // timestamps of this dispatch itself
    hipExtLaunchKernelGGL(kern, grid, block, 0, s, ev0, ev1, 0, xq, sa, wq, sw, M, N, K, kbits, y,
                          acc, tiles_m, tiles_n, gate);
  else
    kern<<<grid, block, 0, s>>>(xq, sa, wq, sw, M, N, K, kbits, y, acc, tiles_m, tiles_n, gate);
  return hipGetLastError();
}

}  // namespace

int gemm_config_count() { return kNumCfgs; }

GemmConfig gemm_config(int index) {
  return GemmConfig{kCfgs[index].bm, kCfgs[index].bn, kCfgs[index].kw};
}

// Estimated time of a configuration: tiles land round-robin on the CUs, so
// the busiest CU runs ceil(tiles / CUs) of them (several at once when they
// fit, sharing its throughput); its time is that count x BM x BN x K / rate.
// The rates are fitted to sweeps of every configuration over the workloads'
// shapes on MI355X; callers that want the measured best use
// tabit_autotune_gemm.
int gemm_config_choose(int M, int N, int K, int num_cus) {
  if (num_cus <= 0) num_cus = 256;
  auto tiles_of = [&](const CfgDesc& c) {
    return (long long)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
  };
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < kNumCfgs; ++i) {
    const CfgDesc& c = kCfgs[i];
    if (c.kw != 1 || c.nst != 2) continue;
    const long long per_cu = (tiles_of(c) + num_cus - 1) / num_cus;
    const double cost = (double)per_cu * c.bm * c.bn / c.rate;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = i;
    }
  }
  // a tile whose workgroups fit in one round over the CUs gives way to its
  // K-split variant (among those whose minimum stage count K reaches) with the
  // fewest stages per group (then the fewest groups):
  // at 64 x 1152 x 1152 three groups of 2 x 2 waves take the masked GEMM from
  // 8.5 to 6.7 us with the weights cold and the bit-plane form from 13.7 to
  // 8.9 us (k = 0), at 512 x 1152 x 4608 (144 tiles) from 22.2 to 15.2 us and at
  // 512 x 1920 x 1920 (240 tiles) from 12.3 to 9.2 us; one-wave groups, even
  // five of them, were slower
  const CfgDesc& b = kCfgs[best];
  if (tiles_of(b) > num_cus) return best;
  const int S = (K + b.rb - 1) / b.rb;
  int pick = best, pick_trips = S, pick_kw = 1;
  for (int i = 0; i < kNumCfgs; ++i) {
    const CfgDesc& c = kCfgs[i];
    if (c.kw == 1 || c.bm != b.bm || c.bn != b.bn || c.rb != b.rb || S < c.min_stages) continue;
    const int trips = (S + c.kw - 1) / c.kw;
    if (trips < pick_trips || (trips == pick_trips && c.kw < pick_kw)) {
      pick = i;
      pick_trips = trips;
      pick_kw = c.kw;
    }
  }
  if (pick != best) return pick;
  // no split taken (for these tiles: fewer than 32 stages): the same tile's
  // deeper ring from its minimum stage count on
  for (int i = 0; i < kNumCfgs; ++i) {
    const CfgDesc& c = kCfgs[i];
    if (c.kw == 1 && c.nst > 2 && c.bm == b.bm && c.bn == b.bn && c.rb == b.rb && S >= c.min_stages)
      return i;
  }
  return best;
}

hipError_t launch_gemm_i8(int cfg, bool bitserial, const int8_t* xq, const float* sa,
                          const int8_t* wq, const float* sw, int M, int N, int K, int kbits,
                          uint16_t* y, int32_t* acc, hipStream_t stream, hipEvent_t ev0,
                          hipEvent_t ev1, const uint8_t* gate) {
#define TABIT_CASE(I, BM, BN, WM, WN, RB, NST, KW, RATE, MS)                                    \
  case I:                                                                                       \
    return launch_cfg<BM, BN, WM, WN, RB, NST, KW>(bitserial, xq, sa, wq, sw, M, N, K, kbits, y, \
                                                   acc, stream, ev0, ev1, gate);
  switch (cfg) {
    TABIT_I8_CONFIGS(TABIT_CASE)
    default: return hipErrorInvalidValue;
  }
#undef TABIT_CASE
}

}  // namespace tabit
