// DMPQ online format selector (6Bit-Diffusion, gist.science summary, section
// 2A): the relative L1 input-output change of a transformer block at step
// t-1, Gamma = sum |out - in| / sum |in|, predicts how sensitive the block's
// linear layers are to quantization at step t; unstable blocks keep INT8,
// stable ones go to 4 bits.  The page prints no predictor coefficients or
// threshold; a linear predictor against a threshold is a per-layer threshold
// on Gamma: INT8 iff Gamma > theta_l.
//
// The decision is written to a device-resident format table, so a captured
// step needs no host round trip: the gated launches of the next step read it.
//
// Summation (the page fixes no order; any order of the n non-negative fp64
// terms is within (n - 1) 2^-53 of the exact sum, relative): terms in fp64
// (|in| exact, out - in one fp64 subtraction); each 16-element chunk summed
// left to right; a row's chunk sums by a butterfly over the lanes and a tree
// over the waves; the row sums by a tree of 1024-leaf groups.  The order is
// fixed, so the same input gives the same Gamma on every run.
#include "tabit_internal.h"

namespace tabit {
namespace {

__device__ __forceinline__ double bf16_to_f64(uint32_t bits16) {
  return (double)__uint_as_float(bits16 << 16);
}

// Sum of one 16-element chunk, left to right, of |out - in| and |in|.
__device__ __forceinline__ void chunk_sums(const uint16_t* in, const uint16_t* out, double& d,
                                           double& a) {
  const uint4* pi = reinterpret_cast<const uint4*>(in);
  const uint4* po = reinterpret_cast<const uint4*>(out);
  const uint4 i0 = pi[0], i1 = pi[1], o0 = po[0], o1 = po[1];
  const uint32_t wi[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
  const uint32_t wo[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t bi = (e & 1) ? (wi[e >> 1] >> 16) : (wi[e >> 1] & 0xFFFFu);
    const uint32_t bo = (e & 1) ? (wo[e >> 1] >> 16) : (wo[e >> 1] & 0xFFFFu);
    const double x = bf16_to_f64(bi), y = bf16_to_f64(bo);
    const double td = fabs(y - x), ta = fabs(x);
    if (e == 0) {
      d = td;
      a = ta;
    } else {
      d = d + td;
      a = a + ta;
    }
  }
}

// Pairwise tree over the lanes of a wave (the same value ends up in every lane).
__device__ __forceinline__ double wave_tree(double v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = v + __shfl_xor(v, off, 64);
  return v;
}

// One workgroup per row: rows[2m] = sum |out - in|, rows[2m + 1] = sum |in|.
// Thread t holds chunks t*CPT .. t*CPT + CPT - 1 (CPT = 2 adds the first tree
// level inside the thread); chunks past the row are zeros.
template <int NT, int CPT>
__global__ void __launch_bounds__(NT)
dmpq_rows_kernel(const uint16_t* __restrict__ xin, const uint16_t* __restrict__ xout, int H,
                 double* __restrict__ rows) {
  constexpr int NW = NT / 64;
  __shared__ double sd[NW], sa[NW];
  const int m = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = H / 16;
  const size_t base = (size_t)m * H;
  double dc[CPT], ac[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid * CPT + i;
    dc[i] = 0.0;
    ac[i] = 0.0;
    if (c < nch) chunk_sums(xin + base + (size_t)c * 16, xout + base + (size_t)c * 16, dc[i], ac[i]);
  }
  double d = dc[0], a = ac[0];
  if constexpr (CPT == 2) {
    d = dc[0] + dc[1];
    a = ac[0] + ac[1];
  }
  d = wave_tree(d);
  a = wave_tree(a);
  if (lane == 0) {
    sd[wave] = d;
    sa[wave] = a;
  }
  __syncthreads();
  if (tid == 0) {
    double vd[NW], va[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      vd[w] = sd[w];
      va[w] = sa[w];
    }
#pragma unroll
    for (int n = NW; n > 1; n >>= 1)
#pragma unroll
      for (int w = 0; w < n / 2; ++w) {
        vd[w] = vd[2 * w] + vd[2 * w + 1];
        va[w] = va[2 * w] + va[2 * w + 1];
      }
    rows[2 * (size_t)m] = vd[0];
    rows[2 * (size_t)m + 1] = va[0];
  }
}

constexpr int FT = 1024;   // leaves per workgroup of a tree level

// One level of the pairwise tree over (sum |out - in|, sum |in|) pairs: group g
// sums leaves [1024g, 1024g + 1024) (zeros past n) with a butterfly and a tree
// over the waves.  Aligned power-of-two groups of a zero-padded pairwise tree
// are its subtrees, so chaining levels reproduces the whole tree.  The last
// level (one group) also forms Gamma and the per-layer decisions.
__global__ void __launch_bounds__(FT)
dmpq_tree_kernel(const double* __restrict__ in, long long n, double* __restrict__ out,
                 const float* __restrict__ theta, int n_layers, uint8_t* __restrict__ fmt,
                 double* __restrict__ gamma_out, int last) {
  constexpr int NW = FT / 64;
  __shared__ double sd[NW], sa[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long leaf = (long long)blockIdx.x * FT + tid;
  double d = 0.0, a = 0.0;
  if (leaf < n) {
    d = in[2 * leaf];
    a = in[2 * leaf + 1];
  }
  d = wave_tree(d);
  a = wave_tree(a);
  if (lane == 0) {
    sd[wave] = d;
    sa[wave] = a;
  }
  __syncthreads();
  if (tid != 0) return;
  double vd[NW], va[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    vd[w] = sd[w];
    va[w] = sa[w];
  }
#pragma unroll
  for (int k = NW; k > 1; k >>= 1)
#pragma unroll
    for (int w = 0; w < k / 2; ++w) {
      vd[w] = vd[2 * w] + vd[2 * w + 1];
      va[w] = va[2 * w] + va[2 * w + 1];
    }
  if (!last) {
    out[2 * blockIdx.x] = vd[0];
    out[2 * blockIdx.x + 1] = va[0];
    return;
  }
  const double num = vd[0], den = va[0];
  double g;
  if (den == 0.0) g = num == 0.0 ? 0.0 : __builtin_huge_val();
  else g = num / den;
  if (gamma_out != nullptr) gamma_out[0] = g;
  for (int l = 0; l < n_layers; ++l) fmt[l] = g > (double)theta[l] ? (uint8_t)0 : (uint8_t)1;
}

int next_pow2(long long v) {
  int p = 0;
  while ((1LL << p) < v) ++p;
  return p;
}

long long groups(long long n) { return (n + FT - 1) / FT; }

}  // namespace

// Row sums, then the partial sums of each tree level (at most 4 levels for
// M < 2^26 rows).
size_t dmpq_workspace_bytes(int M) {
  if (M <= 0) return 0;
  long long pairs = M, n = M;
  while (n > 1) {
    n = groups(n);
    pairs += n;
  }
  return (size_t)(pairs + 1) * 16u;
}

hipError_t launch_dmpq_select(const uint16_t* xin, const uint16_t* xout, int M, int H, double* rows,
                              const float* theta, int n_layers, uint8_t* fmt, double* gamma,
                              hipStream_t s) {
  const int nch = H / 16;
  const int p = 1 << next_pow2(nch);
  if (p <= 64) dmpq_rows_kernel<64, 1><<<M, 64, 0, s>>>(xin, xout, H, rows);
  else if (p == 128) dmpq_rows_kernel<128, 1><<<M, 128, 0, s>>>(xin, xout, H, rows);
  else if (p == 256) dmpq_rows_kernel<256, 1><<<M, 256, 0, s>>>(xin, xout, H, rows);
  else if (p == 512) dmpq_rows_kernel<512, 1><<<M, 512, 0, s>>>(xin, xout, H, rows);
  else if (p == 1024) dmpq_rows_kernel<1024, 1><<<M, 1024, 0, s>>>(xin, xout, H, rows);
  else dmpq_rows_kernel<1024, 2><<<M, 1024, 0, s>>>(xin, xout, H, rows);
  hipError_t e = hipGetLastError();
  double* src = rows;
  long long n = M;
  while (e == hipSuccess) {
    const long long g = groups(n);
    double* dst = src + 2 * n;
    dmpq_tree_kernel<<<(unsigned)g, FT, 0, s>>>(src, n, dst, theta, n_layers, fmt, gamma, g == 1);
    e = hipGetLastError();
    if (g == 1) break;
    src = dst;
    n = g;
  }
  return e;
}

}  // namespace tabit
