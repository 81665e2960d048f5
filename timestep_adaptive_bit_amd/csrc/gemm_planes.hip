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
// Layout: uint32 P[8][K/32][N].  Word P[b][g][n] holds bit b of the 32 weights
// W[n][32g + i]; weight i = 4u + q (u = 0..7, q = 0..3) sits at bit 8q + u.
// Rows n are contiguous for a fixed (plane, group), so a tile's words for one
// plane and K-stage form a few contiguous runs.
//
// GEMM: as the masked INT8 GEMM (K-contiguous int8 activations, LDS stages
// filled by direct global->LDS buffer loads, v_mfma_i32_32x32x32_i8, fused
// dequantization to bf16), except that the weight stage holds the retained
// planes' words and each wave rebuilds its 16-byte weight fragment in
// registers: for every retained plane b one rotate moves the lane's four
// weight bits of each output dword to byte bit b, and one and-or merges them.
// The rebuilt byte is sum_{b >= k} c_b * bit_b = (w >> k) << k exactly
// (c_7 = -128 is the two's-complement sign bit), so the product equals the
// masked GEMM bit for bit with one MFMA per K-step.
#include "tabit_internal.h"
#include "tile_common.h"

namespace tabit {
namespace {

using tile::v4i;
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int RB = 128;        // K bytes per stage = 4 groups of 32 weights
constexpr int GPS = RB / 32;   // groups per stage

// Pack: one thread per (group g, row n), rows fastest so the plane words are
// written coalesced.  Reads the 32 codes W[n][32g .. 32g + 31].
__global__ void __launch_bounds__(256)
pack_planes_kernel(const int8_t* __restrict__ W, int N, int K, uint32_t* __restrict__ P) {
  const int G = K / 32;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)G * N) return;
  const int n = (int)(t % N), g = (int)(t / N);
  const uint4* src = reinterpret_cast<const uint4*>(W + (size_t)n * K + (size_t)g * 32);
  const uint4 lo = src[0], hi = src[1];
  const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};   // d[u]: weights 4u..4u+3
  uint32_t word[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    uint32_t w = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) w |= ((d[u] >> b) & 0x01010101u) << u;   // byte q bit b -> bit 8q + u
    word[b] = w;
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) P[((size_t)b * G + g) * N + n] = word[b];
}

// Copy the retained planes of one K-stage into LDS: slot b (8 slots of
// 16*BN bytes, layout [group][row] words) for b = kbits..7.  Each wave
// instruction fills 1 KB; lane l copies 4 consecutive rows' words of one
// group.  Slots below kbits are never fetched (their lanes read out of range
// and nothing is requested from memory); instructions entirely below kbits
// are skipped.
template <int BN, int NW>
__device__ __forceinline__ void dma_planes(__amdgpu_buffer_rsrc_t rs, int8_t* lds, int n0, int N,
                                           int G, int g0, int kbits, int wave, int lane) {
  constexpr int SLOT = 16 * BN;            // bytes per plane slot
  constexpr int NI = 8 * SLOT / 1024;      // 1 KB instructions per stage
#pragma unroll
  for (int i = 0; i < (NI + NW - 1) / NW; ++i) {
    const int j = i * NW + wave;
    if (j >= NI) break;
    if ((1024 * j + 1023) / SLOT < kbits) continue;   // wave-uniform: every slot dropped
    const int byte = 1024 * j + 16 * lane;
    const int b = byte / SLOT, o = byte % SLOT;
    const int gi = o / (4 * BN), row = (o % (4 * BN)) / 4;
    const bool ok = b >= kbits && g0 + gi < G && n0 + row < N;
    const unsigned off = ok ? (unsigned)((((size_t)b * G + g0 + gi) * N + n0 + row) * 4) : tile::kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (tile::lds_ptr_t)(lds + 1024 * j), 16, off, 0, 0, 0);
  }
}

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM* WN * 64)
gemm_planes_kernel(const int8_t* __restrict__ A, const float* __restrict__ SA,
                   const uint32_t* __restrict__ P, const float* __restrict__ SB, int M, int N,
                   int K, int kbits, uint16_t* __restrict__ Y, int32_t* __restrict__ ACC,
                   int tiles_m, int tiles_n) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int SA_BYTES = BM * RB;
  constexpr int SLOT = 16 * BN;
  constexpr int SP_BYTES = 8 * SLOT;
  constexpr int STAGE = SA_BYTES + SP_BYTES;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold whole 32x32 blocks");
  static_assert((8 * SLOT) % 1024 == 0, "plane slots fill whole 1 KB copies");
  static_assert(2 * STAGE >= BM * BN * 2, "epilogue tile must fit in the LDS stages");
  __shared__ __attribute__((aligned(1024))) int8_t smem[2 * STAGE];

  int tm, tn;
  tile::tile_coords<4>(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int rows_a = min(BM, M - m0);
  const int G = K / 32;
  const auto rsa = tile::make_rsrc(A, (unsigned)M * (unsigned)K);
  const auto rsp = tile::make_rsrc(P, (unsigned)N * (unsigned)K);   // 8 planes x N x K/8 bytes

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16i{};

  const int ra0 = wm * WTM + (lane & 31), rb0 = wn * WTN + (lane & 31);
  const int khalf = lane >> 5;
  const int nk = (K + RB - 1) / RB;
  auto issue = [&](int kt) {
    int8_t* dst = smem + (kt & 1) * STAGE;
    tile::dma_stage<BM, NW, RB>(rsa, dst, m0, rows_a, K, kt * RB, wave, lane);
    dma_planes<BN, NW>(rsp, dst + SA_BYTES, n0, N, G, kt * GPS, kbits, wave, lane);
  };
  issue(0);
  for (int kt = 0; kt < nk; ++kt) {
    tile::wait_vmcnt<0>();
    __syncthreads();   // stage kt visible to all; stage kt-1's buffer is free
    if (kt + 1 < nk) issue(kt + 1);
    const int8_t* sa = smem + (kt & 1) * STAGE;
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(sa + SA_BYTES);
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
        for (int b = kbits; b < 8; ++b) {   // kbits is uniform: a scalar loop
          // word of plane b, group ks, this lane's row; the lane's 16 weights
          // (4t + q for t, q = 0..3) now sit at bit 8q + t
          const uint32_t x = sp[(b * GPS + ks) * BN + rb0 + j * 32] >> (4 * khalf);
          const uint32_t mb = 0x01010101u << b;
          d0 |= __builtin_amdgcn_alignbit(x, x, (0 - b) & 31) & mb;
          d1 |= __builtin_amdgcn_alignbit(x, x, (1 - b) & 31) & mb;
          d2 |= __builtin_amdgcn_alignbit(x, x, (2 - b) & 31) & mb;
          d3 |= __builtin_amdgcn_alignbit(x, x, (3 - b) & 31) & mb;
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

  // 32x32 output layout: lane l, register r holds row (r/4)*8 + (l/32)*4 + r%4, col l%32.
  const int row_w = m0 + wm * WTM, col_w = n0 + wn * WTN;
  if (ACC != nullptr) {
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
    __syncthreads();   // every wave is done reading the last stage
    uint16_t* st = reinterpret_cast<uint16_t*>(smem) + wave * WTM * WTN;
    tile::store_tile32_bf16<WTM, WTN>(st, lane, Y, row_w, col_w, M, N, [&](int i, int j, int r) {
      return tile::bf16_rne(((float)acc[i][j][r] * sa_r[i][r]) * sb_c[j]);
    });
  }
}

struct PlaneCfg {
  int bm, bn, wm, wn;
  float rate;   // relative per-CU throughput when busy
};
// index, BM, BN, WM, WN, rate
#define TABIT_PLANE_CONFIGS(X) \
  X(0, 64, 32, 2, 1, 0.30f)    \
  X(1, 64, 64, 2, 2, 0.45f)    \
  X(2, 128, 128, 2, 2, 1.00f)
#define TABIT_PDESC(I, BM, BN, WM, WN, RATE) {BM, BN, WM, WN, RATE},
constexpr PlaneCfg kPlaneCfgs[] = {TABIT_PLANE_CONFIGS(TABIT_PDESC)};
#undef TABIT_PDESC
constexpr int kNumPlaneCfgs = sizeof(kPlaneCfgs) / sizeof(kPlaneCfgs[0]);

template <int BM, int BN, int WM, int WN>
hipError_t launch_planes_cfg(const int8_t* xq, const float* sa, const uint32_t* wp,
                             const float* sw, int M, int N, int K, int kbits, uint16_t* y,
                             int32_t* acc, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const dim3 grid(tiles_m * tiles_n), block(WM * WN * 64);
  auto kern = gemm_planes_kernel<BM, BN, WM, WN>;
  if (ev0 != nullptr || ev1 != nullptr)
    hipExtLaunchKernelGGL(kern, grid, block, 0, s, ev0, ev1, 0, xq, sa, wp, sw, M, N, K, kbits, y,
                          acc, tiles_m, tiles_n);
  else
    kern<<<grid, block, 0, s>>>(xq, sa, wp, sw, M, N, K, kbits, y, acc, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_planes(const int8_t* wq, int N, int K, uint32_t* planes, hipStream_t s) {
  const long long threads = (long long)(K / 32) * N;
  const int grid = (int)((threads + 255) / 256);
  pack_planes_kernel<<<grid, 256, 0, s>>>(wq, N, K, planes);
  return hipGetLastError();
}

int plane_config_count() { return kNumPlaneCfgs; }

GemmConfig plane_config(int index) {
  return GemmConfig{kPlaneCfgs[index].bm, kPlaneCfgs[index].bn, 1};
}

// Tiles land round-robin on the CUs, so the busiest CU runs ceil(tiles / CUs)
// of them; its time is that count times the tile's work over the tile's rate.
int plane_config_choose(int M, int N, int K, int num_cus) {
  (void)K;
  if (num_cus <= 0) num_cus = 256;
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < kNumPlaneCfgs; ++i) {
    const PlaneCfg& c = kPlaneCfgs[i];
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

hipError_t launch_gemm_planes(int cfg, const int8_t* xq, const float* sa, const uint32_t* wp,
                              const float* sw, int M, int N, int K, int kbits, uint16_t* y,
                              int32_t* acc, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
#define TABIT_PCASE(I, BM, BN, WM, WN, RATE) \
  case I:                                   \
    return launch_planes_cfg<BM, BN, WM, WN>(xq, sa, wp, sw, M, N, K, kbits, y, acc, stream, ev0, ev1);
  switch (cfg) {
    TABIT_PLANE_CONFIGS(TABIT_PCASE)
    default: return hipErrorInvalidValue;
  }
#undef TABIT_PCASE
}

}  // namespace tabit
