// Tile-level helpers shared by the INT8 and MXFP4 GEMM kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tabit {
namespace tile {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr unsigned kOOB = 0x80000000u;    // buffer offset past any operand: loads return 0
constexpr int kRsrcFlags = 0x00020000;    // raw buffer descriptor word 3 for gfx9-family parts

// LDS rows of RB bytes (64 or 128) hold RB/16 16-byte chunks; chunk c of row r
// sits at slot c ^ swz<RB>(r).  The LDS serves 16 lanes x 16 bytes per clock
// from a 256-byte bank window; MFMA operand reads have 16 consecutive lanes on
// 16 consecutive rows at one logical chunk, and the swizzle sends those 16 rows
// to 16 distinct 16-byte bank groups (the window holds 256/RB rows, the XOR
// separates the rows that share a window position).  DMA writes fill whole
// 1 KB blocks and are conflict-free by construction.
template <int RB>
__device__ __forceinline__ int swz(int r) {
  if constexpr (RB == 128) return (r & 7) ^ ((r >> 3) & 1);
  else return (r >> 2) & 3;
}
template <int RB = 128>
__device__ __forceinline__ int lds_off(int r, int c) { return r * RB + ((c ^ swz<RB>(r)) << 4); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kRsrcFlags);
}

// Direct global->LDS copy of one stage: ROWS rows x RB bytes starting at byte
// kb0 of each row.  Each wave instruction fills one 1 KB LDS block (1024/RB
// rows); lane l writes slot l % (RB/16) of row l / (RB/16) of that block, so it
// fetches the logical chunk the swizzle places there.  Rows past rows_valid and
// chunks past row_bytes read out of range and land as zeros.  Block j goes to
// wave j % NWAVES; when the blocks do not split evenly, the first waves take
// one more (callers then wait for all of a stage's copies at once).
template <int ROWS, int NWAVES, int RB = 128>
__device__ __forceinline__ void dma_stage(__amdgpu_buffer_rsrc_t rs, int8_t* lds, int row0,
                                          int rows_valid, int row_bytes, int kb0, int wave,
                                          int lane) {
  constexpr int CPR = RB / 16;           // chunks per row
  constexpr int RPB = 1024 / RB;         // rows per 1 KB block
  constexpr int BLOCKS = ROWS / RPB;
  static_assert(ROWS % RPB == 0, "tile rows must fill whole 1 KB blocks");
#pragma unroll
  for (int i = 0; i < (BLOCKS + NWAVES - 1) / NWAVES; ++i) {
    const int j = i * NWAVES + wave;
    if (BLOCKS % NWAVES != 0 && j >= BLOCKS) break;   // wave-uniform
    const int r = RPB * j + lane / CPR;
    const int c = (lane % CPR) ^ swz<RB>(r);
    const int gk = kb0 + c * 16;
    const unsigned off =
        (r < rows_valid && gk < row_bytes) ? (unsigned)((row0 + r) * row_bytes + gk) : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(lds + j * 1024), 16, off, 0, 0, 0);
  }
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left at their maxima (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ void wait_vmcnt0() { wait_vmcnt<0>(); }

// Workgroup barrier for a ring of LDS stages filled by buffer loads into LDS.
// __syncthreads() (its release fence) also waits for every vector-memory load
// in flight, those copies included, which would drain the stages the ring
// keeps in flight.  Here each wave waits only for its own LDS reads and writes
// (a buffer's last readers are done before anyone refills it); the copies a
// stage needs are waited for by count (wait_vmcnt) before the barrier.  The
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maxima
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Logical tile of this workgroup.  Dispatch hands consecutive workgroup ids to
// the 8 XCDs round-robin, and each XCD has its own L2; undo that so every XCD
// works on a contiguous range of logical tiles, then walk tiles in groups of
// GROUP_M tile-rows (column-major inside a group) so concurrently running
// tiles share A rows and B columns in L2.
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

// Epilogue of a wave tile WTM x WTN through its LDS staging `st`: MFMA-layout
// writes of the bf16 values, one barrier, then row-contiguous 16-byte global
// stores.  For the 32x32 MFMA output layout: fragment (i, j) is a 32 x 32
// block; lane l, register r holds row (r/4)*8 + (l/32)*4 + r%4, column l%32.
// `val(i, j, r)` gives the bf16 of fragment (i, j), register r.  The
// chunk swizzle XORs within aligned groups of SW chunks, SW the largest power
// of two dividing the row's chunk count (12 chunks of a 96-wide tile: 4).  The
// global stores are nontemporal (1.6-5% faster on MI355X than plain stores for
// the 128 x 64 and 256 x 256 tiles).
// `active` = false: the wave only takes part in the barrier (for workgroups
// where some waves hold no output).
template <int WTM, int WTN, typename F>
__device__ __forceinline__ void store_tile32_bf16(uint16_t* st, int lane, uint16_t* __restrict__ Y,
                                                  int row0, int col0, int M, int N, F val,
                                                  bool active = true) {
  constexpr int FM = WTM / 32, FN = WTN / 32, CH = WTN / 8, SW = CH & -CH;
  if (active) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int lc = j * 32 + (lane & 31);
          const int ch = (lc >> 3) ^ (lr & (SW - 1));
          st[lr * WTN + ch * 8 + (lc & 7)] = val(i, j, r);
        }
  }
  __syncthreads();
  if (!active) return;
#pragma unroll
  for (int it = 0; it < WTM * CH / 64; ++it) {
    const int idx = it * 64 + lane;
    const int lr = idx / CH, ch = idx % CH;
    const int gm = row0 + lr, gn = col0 + ch * 8;
    const v4u v = *reinterpret_cast<const v4u*>(st + lr * WTN + ((ch ^ (lr & (SW - 1))) * 8));
    // streaming store: the tile is written once and read by the next kernel
    if (gm < M && gn < N) __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(Y + (size_t)gm * N + gn));
  }
}

}  // namespace tile
}  // namespace tabit
