// Plane-major storage of the shared INT8 weight buffer, and the GEMM that
// streams only the bit-planes a layer-step keeps.
//
// TASQ (gist.science summary, section 2 "Metodologia", Temporal-Precision
// Engine): activation planes stay on chip while only the weight bit-planes
// selected for the layer and step are fetched, which cuts plane fetches from
// 2LR to L + R.  On a fixed-precision matrix core the arithmetic does not
// shrink with the bit width (same summary, section 5), but the memory traffic
// can: the same 8 bits per weight are stored plane by plane, so a step with
// mask k reads (8 - k)/8 of the buffer and never touches the k dropped planes.
// The storage is the same size as the INT8 buffer (one copy, no per-step
// copies).
//
// Layout: uint32 P[8][S][N][4], S = ceil(K/128).  Word P[b][s][n][j] holds bit
// b of the 32 weights W[n][128s + 32j + i]; weight i = 4u + q (u = 0..7,
// q = 0..3) sits at bit 8q + u; words past K are zero.  For one plane and one
// 128-weight K-stage a row's four words are 16 contiguous bytes and a tile's
// rows are one contiguous run, so a plane's stage is copied with full 16-byte
// lanes and read back from LDS with one 16-byte read per lane.
//
// GEMM: as the masked INT8 GEMM (K-contiguous int8 activations, LDS stages
// filled by direct global->LDS buffer loads, v_mfma_i32_32x32x32_i8, fused
// dequantization to bf16), except that the weight stage holds the retained
// planes' words and each wave rebuilds its 16-byte weight fragment in
// registers: for every retained plane b one rotate moves the lane's four
// weight bits of each output dword to byte bit b, and one and-or merges them
// (planes unrolled, dropped planes skipped by a uniform branch).
// The rebuilt byte is sum_{b >= k} c_b * bit_b = (w >> k) << k exactly
// (c_7 = -128 is the two's-complement sign bit), so the product equals the
// masked GEMM bit for bit with one MFMA per K-step.
//
// K split inside the workgroup (KW > 1), for few-token shapes whose tiles
// leave most CUs idle: KW groups of WM x WN waves each walk a contiguous range
// of the K stages through their own LDS ring, then groups 1..KW-1 hand their
// int32 accumulators to group 0 through LDS (integer sums: the result is the
// unsplit one bit for bit) and group 0 runs the epilogue.  Every wave takes
// part in every barrier.
#include "tabit_internal.h"
#include "tile_common.h"

namespace tabit {
namespace {

using tile::v4i;
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int RB = 128;        // K bytes per stage = 4 groups of 32 weights
constexpr int GPS = RB / 32;   // groups per stage

// Pack: one thread per (stage s, row n, word j), j fastest, so both the 32
// codes a thread reads and the words the threads write are contiguous.
__global__ void __launch_bounds__(256)
pack_planes_kernel(const int8_t* __restrict__ W, int N, int K, uint32_t* __restrict__ P) {
  const int S = (K + RB - 1) / RB;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)S * N * GPS) return;
  const int j = (int)(t % GPS);
  const int n = (int)((t / GPS) % N);
  const int st = (int)(t / ((long long)GPS * N));
  const int k0 = st * RB + 32 * j;
  uint32_t word[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (k0 < K) {
    const uint4* src = reinterpret_cast<const uint4*>(W + (size_t)n * K + k0);
    const uint4 lo = src[0], hi = src[1];
    const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};   // d[u]: weights 4u..4u+3
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      uint32_t w = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) w |= ((d[u] >> b) & 0x01010101u) << u;   // byte q bit b -> bit 8q + u
      word[b] = w;
    }
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) P[(((size_t)b * S + st) * N + n) * GPS + j] = word[b];
}

// Copy the retained planes of K-stage `st` into LDS: slot b (8 slots of
// 16*BN bytes, one 16-byte row of 4 words per tile row) for b = kbits..7.
// Each wave instruction fills 1 KB (64 rows of one plane, or two planes'
// slots when BN = 32).  Lanes of dropped planes read out of range, so nothing
// is requested from memory for them; the instructions are still issued so
// every wave has the same, compile-time number of copies in flight.
template <int BN, int NW>
__device__ __forceinline__ void dma_planes(__amdgpu_buffer_rsrc_t rs, int8_t* lds, int n0, int N,
                                           int S, int st, int kbits, int wave, int lane) {
  constexpr int SLOT = 16 * BN;            // bytes per plane slot
  constexpr int NI = 8 * SLOT / 1024;      // 1 KB instructions per stage
#pragma unroll
  for (int i = 0; i < (NI + NW - 1) / NW; ++i) {
    const int j = i * NW + wave;
    if (j >= NI) break;
    const int byte = 1024 * j + 16 * lane;
    const int b = byte / SLOT, row = (byte % SLOT) / 16;
    const bool ok = b >= kbits && n0 + row < N;
    const unsigned off = ok ? (unsigned)((((size_t)b * S + st) * N + n0 + row) * 16) : tile::kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (tile::lds_ptr_t)(lds + 1024 * j), 16, off, 0, 0, 0);
  }
}

template <int BM, int BN, int WM, int WN, int NST, int KW>
__global__ void __launch_bounds__(WM* WN * KW * 64)
gemm_planes_kernel(const int8_t* __restrict__ A, const float* __restrict__ SA,
                   const uint32_t* __restrict__ P, const float* __restrict__ SB, int M, int N,
                   int K, int kbits, uint16_t* __restrict__ Y, int32_t* __restrict__ ACC,
                   int tiles_m, int tiles_n, const uint8_t* __restrict__ gate) {
  if (gate != nullptr && *gate != 0) return;   // device-selected format is not INT8
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int SA_BYTES = BM * RB;
  constexpr int SLOT = 16 * BN;
  constexpr int SP_BYTES = 8 * SLOT;
  constexpr int STAGE = SA_BYTES + SP_BYTES;
  constexpr int NI = SP_BYTES / 1024;                         // plane copies per stage
  constexpr int DPW = SA_BYTES / 1024 / NW + (NI + NW - 1) / NW;   // copies per wave per stage
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold whole 32x32 blocks");
  static_assert(SP_BYTES % 1024 == 0 && NI % NW == 0, "plane copies split evenly over the waves");
  static_assert(NST >= 2 && NST <= 4, "2 to 4 LDS stages");
  static_assert(NST * STAGE >= BM * BN * 2, "epilogue tile must fit in the LDS stages");
  static_assert(KW >= 1 && (KW - 1) * BM * BN * 4 <= KW * NST * STAGE,
                "the K groups' partial accumulators must fit in the LDS stages");
  static_assert(NW * KW * 64 <= 1024, "at most 1024 threads per workgroup");
  __shared__ __attribute__((aligned(1024))) int8_t smem[KW * NST * STAGE];

  int tm, tn;
  tile::tile_coords<4>(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  // K group and wave within it (compile-time 0 and the wave id without a split)
  const int group = KW > 1 ? (tid >> 6) / NW : 0;
  const int wave = KW > 1 ? (tid >> 6) % NW : (tid >> 6), lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  int8_t* ring = smem + group * NST * STAGE;
  const int rows_a = min(BM, M - m0);
  const int S = (K + RB - 1) / RB;
  const auto rsa = tile::make_rsrc(A, (unsigned)M * (unsigned)K);
  const auto rsp = tile::make_rsrc(P, (unsigned)S * 128u * (unsigned)N);   // 8 planes x S x N x 16 bytes

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16i{};

  const int ra0 = wm * WTM + (lane & 31), rb0 = wn * WTN + (lane & 31);
  const int khalf = lane >> 5;
  // this group's stages [kt0, kt0 + nk); every group runs `trips` iterations
  const int trips = KW > 1 ? (S + KW - 1) / KW : S;
  const int kt0 = KW > 1 ? group * trips : 0;
  const int nk = KW > 1 ? max(0, min(S - kt0, trips)) : S;
  // rotate amounts (t - b + 4*khalf) mod 32 for t - b = -7..3: bit 8q + 4*khalf + t
  // of a word (this lane's weight 4t + q) moves to bit 8q + b
  int rot[11];
#pragma unroll
  for (int d = 0; d < 11; ++d) rot[d] = (d - 7 + 4 * khalf) & 31;
  auto issue = [&](int it) {
    int8_t* dst = ring + (it % NST) * STAGE;
    tile::dma_stage<BM, NW, RB>(rsa, dst, m0, rows_a, K, (kt0 + it) * RB, wave, lane);
    dma_planes<BN, NW>(rsp, dst + SA_BYTES, n0, N, S, kt0 + it, kbits, wave, lane);
  };
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < nk) issue(st);
  for (int kt = 0; kt < trips; ++kt) {
    // stage kt has landed once at most (stages issued after it) x DPW copies are pending
    const int ahead = min(NST - 2, nk - 1 - kt);
    if (NST >= 4 && ahead >= 2) tile::wait_vmcnt<(NST >= 4 ? 2 : 0) * DPW>();
    else if (NST >= 3 && ahead >= 1) tile::wait_vmcnt<(NST >= 3 ? 1 : 0) * DPW>();
    else tile::wait_vmcnt<0>();
    tile::lds_barrier();   // stage kt visible to all; stage kt-1's buffer is free
    if constexpr (KW > 1) {
      if (kt >= nk) continue;   // this group's range is done (the barrier above still counts it)
    }
    if (kt + NST - 1 < nk) issue(kt + NST - 1);
    const int8_t* sa = ring + (kt % NST) * STAGE;
    const int8_t* sp = sa + SA_BYTES;
    // this lane's row of every retained plane: 4 words = the stage's 4 K-steps
    // (read as a vector type: a HIP uint4 struct load loses the access's alias
    // information, and the compiler then orders it after every copy in flight)
    tile::v4u pw[FN][8];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int b = 0; b < 8; ++b)
        if (b >= kbits) pw[j][b] = *reinterpret_cast<const tile::v4u*>(sp + (b * BN + rb0 + j * 32) * 16);
#pragma unroll
    for (int ks = 0; ks < GPS; ++ks) {
      v4i a[FM], bw[FN];
      const int c = ks * 2 + khalf;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const v4i*>(sa + tile::lds_off<RB>(ra0 + i * 32, c));
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        uint32_t d0 = 0, d1 = 0, d2 = 0, d3 = 0;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          if (b < kbits) continue;   // uniform: dropped planes are neither read nor merged
          const uint32_t x = pw[j][b][ks];
          const uint32_t mb = 0x01010101u << b;
          d0 |= __builtin_amdgcn_alignbit(x, x, rot[0 - b + 7]) & mb;
          d1 |= __builtin_amdgcn_alignbit(x, x, rot[1 - b + 7]) & mb;
          d2 |= __builtin_amdgcn_alignbit(x, x, rot[2 - b + 7]) & mb;
          d3 |= __builtin_amdgcn_alignbit(x, x, rot[3 - b + 7]) & mb;
        }
        bw[j] = v4i{(int)d0, (int)d1, (int)d2, (int)d3};
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], bw[j], acc[i][j], 0, 0, 0);
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

  // 32x32 output layout: lane l, register r holds row (r/4)*8 + (l/32)*4 + r%4, col l%32.
  const int row_w = m0 + wm * WTM, col_w = n0 + wn * WTN;
  if (ACC != nullptr && out) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gm = row_w + i * 32 + (r >> 2) * 8 + khalf * 4 + (r & 3);
          const int gn = col_w + j * 32 + (lane & 31);
          if (gm < M && gn < N) ACC[(size_t)gm * N + gn] = acc[i][j][r];
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
    __syncthreads();   // every wave is done reading the last stage (or the partial sums)
    uint16_t* st = reinterpret_cast<uint16_t*>(smem) + wave * WTM * WTN;
    tile::store_tile32_bf16<WTM, WTN>(st, lane, Y, row_w, col_w, M, N, [&](int i, int j, int r) {
      return tile::bf16_rne(((float)acc[i][j][r] * sa_r[i][r]) * sb_c[j]);
    }, out);
  }
}

struct PlaneCfg {
  int bm, bn, wm, wn, nst, kw;
  float rate;   // relative per-CU throughput when busy
};
// Rates fitted to a graph-replayed sweep (k = 0 and 4, 64 to 4096 tokens):
// the 128 x 64 tile is as fast per tile element as 128 x 128 on MI355X (the
// byte rebuild, not the fill, bounds both); 8- and 16-wave tiles were slower
// (more waves compete for the rebuild's VALU slots).
// index, BM, BN, WM, WN, LDS stages, K groups, rate
#define TABIT_PLANE_CONFIGS(X)      \
  X(0, 64, 32, 1, 1, 4, 1, 0.40f)   \
  X(1, 64, 64, 1, 2, 2, 1, 0.80f)   \
  X(2, 128, 64, 1, 2, 2, 1, 1.00f)  \
  X(3, 128, 128, 2, 2, 2, 1, 1.00f) \
  X(4, 64, 32, 1, 1, 2, 3, 0.30f)   \
  X(5, 64, 32, 1, 1, 2, 5, 0.30f)   \
  X(6, 64, 64, 1, 2, 2, 3, 0.45f)
#define TABIT_PDESC(I, BM, BN, WM, WN, NST, KW, RATE) {BM, BN, WM, WN, NST, KW, RATE},
constexpr PlaneCfg kPlaneCfgs[] = {TABIT_PLANE_CONFIGS(TABIT_PDESC)};
#undef TABIT_PDESC
constexpr int kNumPlaneCfgs = sizeof(kPlaneCfgs) / sizeof(kPlaneCfgs[0]);

template <int BM, int BN, int WM, int WN, int NST, int KW>
hipError_t launch_planes_cfg(const int8_t* xq, const float* sa, const uint32_t* wp,
                             const float* sw, int M, int N, int K, int kbits, uint16_t* y,
                             int32_t* acc, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                             const uint8_t* gate) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const dim3 grid(tiles_m * tiles_n), block(WM * WN * KW * 64);
  auto kern = gemm_planes_kernel<BM, BN, WM, WN, NST, KW>;
  if (ev0 != nullptr || ev1 != nullptr)
    hipExtLaunchKernelGGL(kern, grid, block, 0, s, ev0, ev1, 0, xq, sa, wp, sw, M, N, K, kbits, y,
                          acc, tiles_m, tiles_n, gate);
  else
    kern<<<grid, block, 0, s>>>(xq, sa, wp, sw, M, N, K, kbits, y, acc, tiles_m, tiles_n, gate);
  return hipGetLastError();
}

}  // namespace

size_t planes_bytes(int N, int K) { return (size_t)((K + RB - 1) / RB) * 128u * (size_t)N; }

hipError_t launch_pack_planes(const int8_t* wq, int N, int K, uint32_t* planes, hipStream_t s) {
  const long long threads = (long long)((K + RB - 1) / RB) * N * GPS;
  const int grid = (int)((threads + 255) / 256);
  pack_planes_kernel<<<grid, 256, 0, s>>>(wq, N, K, planes);
  return hipGetLastError();
}

int plane_config_count() { return kNumPlaneCfgs; }

GemmConfig plane_config(int index) {
  return GemmConfig{kPlaneCfgs[index].bm, kPlaneCfgs[index].bn, kPlaneCfgs[index].kw};
}

// Tiles land round-robin on the CUs, so the busiest CU runs ceil(tiles / CUs)
// of them; its time is that count times the tile's work over the tile's rate
// (one K group per workgroup).  When the chosen tile's workgroups fit in one
// round over the CUs, the variant of the same tile with the most K groups that
// cuts the stages each group walks (fewest trips, then fewest groups) replaces
// it: at 64 x 1152 x 1152 five groups take 17.3 us down to 7.9 (k = 0), at
// 256 x 1152 x 1152 (144 tiles) 16.9 down to 8.2.
int plane_config_choose(int M, int N, int K, int num_cus) {
  if (num_cus <= 0) num_cus = 256;
  auto tiles_of = [&](const PlaneCfg& c) {
    return (long long)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
  };
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < kNumPlaneCfgs; ++i) {
    const PlaneCfg& c = kPlaneCfgs[i];
    if (c.kw != 1) continue;
    const long long per_cu = (tiles_of(c) + num_cus - 1) / num_cus;
    const double cost = (double)per_cu * c.bm * c.bn / c.rate;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = i;
    }
  }
  const PlaneCfg& b = kPlaneCfgs[best];
  if (tiles_of(b) > num_cus) return best;
  const int S = (K + RB - 1) / RB;
  int pick = best, pick_trips = S, pick_kw = 1;
  for (int i = 0; i < kNumPlaneCfgs; ++i) {
    const PlaneCfg& c = kPlaneCfgs[i];
    if (c.kw == 1 || c.bm != b.bm || c.bn != b.bn) continue;
    const int trips = (S + c.kw - 1) / c.kw;
    if (trips < pick_trips || (trips == pick_trips && c.kw < pick_kw)) {
      pick = i;
      pick_trips = trips;
      pick_kw = c.kw;
    }
  }
  return pick;
}

hipError_t launch_gemm_planes(int cfg, const int8_t* xq, const float* sa, const uint32_t* wp,
                              const float* sw, int M, int N, int K, int kbits, uint16_t* y,
                              int32_t* acc, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1,
                              const uint8_t* gate) {
#define TABIT_PCASE(I, BM, BN, WM, WN, NST, KW, RATE) \
  case I:                                            \
    return launch_planes_cfg<BM, BN, WM, WN, NST, KW>(xq, sa, wp, sw, M, N, K, kbits, y, acc,   \
                                                      stream, ev0, ev1, gate);
  switch (cfg) {
    TABIT_PLANE_CONFIGS(TABIT_PCASE)
    default: return hipErrorInvalidValue;
  }
#undef TABIT_PCASE
}

}  // namespace tabit
