// sgemm_kernels.hpp -- the gfx950 SGEMM kernel template.
//
// One workgroup computes one BM x BN tile of C = alpha*A*B + beta*C (the block
// tile of "Warp Tiling: A Third Level of Tiling", section "The Kernel"); each
// 64-lane wave owns a WM x WN warp tile split into WMITER x WNITER sub-tiles.
// The K loop walks BK-wide slices:
//
//   prologue: stage slice 0 into LDS buffer 0, barrier
//   for each slice kt:
//       issue the global loads of slice kt+1 into registers
//       inner product over buffer kt&1 (VALU outer products or MFMA blocks)
//       write the registers of slice kt+1 into buffer (kt+1)&1
//       barrier
//   epilogue: C = alpha*acc + beta*C for in-range elements only
//
// With two LDS buffers one barrier per slice is enough: a buffer is only
// rewritten one iteration after every wave has passed the barrier that ended
// its last use (the page "Shared Memory Tiling" explains why a single buffer
// needs a barrier on both sides of the inner product).
//
// With the direct-LDS option (MFMA 32x32x2, float4 variant) the loads of
// slice kt+1 write the other LDS stage themselves: no staging registers and no
// LDS stores; each wave waits for its own loads (vmcnt) before the barrier.
//
// Operands are read through buffer resources rebuilt per slice, so every load
// is range-checked by the hardware; elements outside the logical M x K and
// K x N windows are masked by giving them an offset past the resource's end,
// which returns zero without touching memory.  The VEC variant moves float4s
// and needs K % 4 == N % 4 == 0, lda % 4 == ldb % 4 == ldc % 4 == 0 and
// 16-byte aligned pointers (checked by the host); the scalar variant moves
// single floats with the same staging map and LDS layout and accepts any
// shape and leading dimension.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_maps.hpp"

namespace fp32gemm {

struct KernelArgs {
  const float* A;
  const float* B;
  float* C;
  long long lda, ldb, ldc;
  int M, N, K;
  int tiles_m, tiles_n;  // ceil(M / BM), ceil(N / BN)
  int group_m;           // tile rows per group of the XCD-aware order
  int nk;                // K slices per tile: ceil(K / BK)
  int tiles_full;        // tiles computed whole, one workgroup each
  int splits;            // K segments of each remaining tile (1 = no split)
  float alpha, beta;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Buffer resources never describe more than kMaxRecords bytes; a masked
// element is loaded from kMaskedOffset, which is therefore always out of
// range and reads as zero.
constexpr long long kMaxRecords = kMaxBufferBytes;
constexpr int kMaskedOffset = 0x7FFFFFF0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float* base, long long bytes) {
  const long long b = bytes < 0 ? 0 : (bytes > kMaxRecords ? kMaxRecords : bytes);
  // Word 3 = 0x00020000: 32-bit data format, raw (unswizzled, stride 0) buffer.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), static_cast<short>(0),
                                           static_cast<int>(b), 0x00020000);
}

// A resource of `bytes` bytes (0 <= bytes <= kMaxRecords, which the caller
// guarantees).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_exact(const float* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), static_cast<short>(0), bytes,
                                           0x00020000);
}

__device__ __forceinline__ f32x4 buffer_load4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float buffer_load1(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}

__device__ __forceinline__ void buffer_store1(__amdgpu_buffer_rsrc_t r, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, off, 0, 0);
}

template <class Cfg>
struct Staged {
  f32x4 a[Cfg::PASSES_A];
  f32x4 b[Cfg::PASSES_B];
};

// Global -> registers for the slice starting at k0.
template <class Cfg, bool VEC>
__device__ __forceinline__ void stage_load(const KernelArgs& p, int row0, int col0, int k0, int t,
                                           Staged<Cfg>& s) {
  constexpr Geom g = make_geom(Cfg::tile);
  const int lda = static_cast<int>(p.lda), ldb = static_cast<int>(p.ldb);

  const int rows = min(g.BM, p.M - row0);
  const float* abase = p.A + static_cast<long long>(row0) * p.lda + k0;
  const auto ra = make_rsrc(abase, (static_cast<long long>(rows - 1) * p.lda + (p.K - k0)) * 4);
#pragma unroll
  for (int ps = 0; ps < g.PASSES_A; ++ps) {
    const int m = stage_a_row(g, t, ps), c = 4 * stage_a_kq(g, t);
    if constexpr (VEC) {
      const bool ok = (m < rows) && (k0 + c < p.K);
      s.a[ps] = buffer_load4(ra, ok ? (m * lda + c) * 4 : kMaskedOffset);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = (m < rows) && (k0 + c + e < p.K);
        s.a[ps][e] = buffer_load1(ra, ok ? (m * lda + c + e) * 4 : kMaskedOffset);
      }
    }
  }

  const int krows = min(g.BK, p.K - k0);
  const float* bbase = p.B + static_cast<long long>(k0) * p.ldb + col0;
  const auto rb = make_rsrc(bbase, (static_cast<long long>(krows - 1) * p.ldb + (p.N - col0)) * 4);
#pragma unroll
  for (int ps = 0; ps < g.PASSES_B; ++ps) {
    const int k = stage_b_row(g, t, ps), c = 4 * stage_b_nq(g, t);
    if constexpr (VEC) {
      const bool ok = (k < krows) && (col0 + c < p.N);
      s.b[ps] = buffer_load4(rb, ok ? (k * ldb + c) * 4 : kMaskedOffset);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = (k < krows) && (col0 + c + e < p.N);
        s.b[ps][e] = buffer_load1(rb, ok ? (k * ldb + c + e) * 4 : kMaskedOffset);
      }
    }
  }
}

// Registers -> LDS stage: A scattered transposed into As[k][m], B as float4
// rows of Bs[k][n].
template <class Cfg>
__device__ __forceinline__ void stage_store(float* stage, int t, const Staged<Cfg>& s) {
  constexpr Geom g = make_geom(Cfg::tile);
#pragma unroll
  for (int ps = 0; ps < g.PASSES_A; ++ps) {
    const int m = stage_a_row(g, t, ps), c = 4 * stage_a_kq(g, t);
#pragma unroll
    for (int e = 0; e < 4; ++e) stage[as_index(g, c + e, m)] = s.a[ps][e];
  }
#pragma unroll
  for (int ps = 0; ps < g.PASSES_B; ++ps) {
    const int k = stage_b_row(g, t, ps), c = 4 * stage_b_nq(g, t);
    *reinterpret_cast<f32x4*>(&stage[bs_index(g, k, c)]) = s.b[ps];
  }
}

// ---- direct-LDS staging --------------------------------------------------

// LDS (address space 3) pointer; a C-style cast from a generic pointer into
// a __shared__ array is an address-space cast.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Direct-LDS slices run partial-first: with nk = ceil(K / BK) slices and
// r = K - (nk - 1) * BK (1 <= r <= BK; r = 0 when K = 0), slice 0 covers
// k in [0, r) and slice s >= 1 covers [r + (s - 1) * BK, r + s * BK).  Only
// slice 0 needs a mask along K (in the prologue); every slice the loop
// loads is whole, or lies past K entirely and gets an empty resource.
__device__ __forceinline__ int tail_width(const KernelArgs& p, int BK) {
  return p.nk > 0 ? p.K - (p.nk - 1) * BK : 0;
}
__device__ __forceinline__ int slice_k0(int kt, int r, int BK) {
  return kt == 0 ? 0 : r + (kt - 1) * BK;
}

// Per-lane byte offsets of this wave's direct-LDS instructions from the slice
// origin (A[row0][k0], B[k0][col0]); they do not change from slice to slice.
// Rows of A past M need no mask: they lie past the end of the slice's buffer
// resource (lda >= K), so they load as zero without being read.  Columns of B
// past N would fall inside the resource (the next row's elements or ldb
// padding), so their offsets are masked here, once.
//
// The tile's operand origins and resource extents are also fixed here, so a
// slice's resources cost a few scalar additions: every slice after the first
// is either whole (k0 + BK <= K) or lies past K, so the A resource of the
// slice at k0 spans a_ext + (K - k0) * 4 bytes (the rows above the last one,
// then the last row's elements from k0 to K) and the B resource b_ext bytes
// (BK - 1 rows, then the in-range columns of the last one).  Both are below
// kMaxBufferBytes (lda, ldb >= K, N and at most kMaxLeadingDim; BM, BK <=
// kMaxTileRows), so they fit in 32 bits.
//
// VA: 16-byte loads for both operands (4-byte loads otherwise); the hybrid
// kernels' first K slice loads A 4 bytes per lane (dma_first_slice's A1S).
template <class Cfg, bool VA>
struct DmaLanes {
  static constexpr Geom g = make_geom(Cfg::tile);
  static constexpr int FPL = VA ? 4 : 1;
  // The VALU path loads its transposed A 4 bytes per lane in both variants.
  static constexpr int FPL_A = Cfg::PATH == kPathValu ? 1 : VA ? 4 : 1;
  int a_off[dma_ops_a(g, FPL_A)];
  int b_off[dma_ops_b(g, FPL)];
  const float* a_row;  // &A[row0][0]
  const float* b_col;  // &B[0][col0]
  int a_ext, b_ext;
};

template <class Cfg, bool VA>
__device__ __forceinline__ void dma_setup(const KernelArgs& p, int row0, int col0, int wave,
                                          int lane, DmaLanes<Cfg, VA>& d) {
  constexpr Geom g = make_geom(Cfg::tile);
  constexpr int FPL = DmaLanes<Cfg, VA>::FPL, FPL_A = DmaLanes<Cfg, VA>::FPL_A;
  static_assert(g.BM <= kMaxTileRows && g.BK <= kMaxTileRows, "resource extents need 32 bits");
  const int lda = static_cast<int>(p.lda), ldb = static_cast<int>(p.ldb);
  const int cols = p.N - col0;
  const int rows = min(g.BM, p.M - row0);
  d.a_row = p.A + static_cast<long long>(row0) * p.lda;
  d.b_col = p.B + col0;
  d.a_ext = static_cast<int>(static_cast<long long>(rows - 1) * p.lda * 4);
  d.b_ext = static_cast<int>((static_cast<long long>(g.BK - 1) * p.ldb + cols) * 4);
#pragma unroll
  for (int j = 0; j < dma_ops_a(g, FPL_A); ++j) {
    const MK s = Cfg::PATH == kPathValu ? dma_at_src(g, dma_op(g, wave, j), lane)
                                        : dma_a_src(g, dma_op(g, wave, j), lane, FPL_A);
    d.a_off[j] = (s.m * lda + s.k) * 4;
  }
#pragma unroll
  for (int j = 0; j < dma_ops_b(g, FPL); ++j) {
    const KN s = dma_b_src(g, dma_op(g, wave, j), lane, FPL);
    // A float4 that starts before column N may cross it; what it brings past
    // N feeds only outputs the epilogue never stores.
    d.b_off[j] = s.n < cols ? (s.k * ldb + s.n) * 4 : kMaskedOffset;
  }
}

template <bool VEC>
__device__ __forceinline__ void dma_load(__amdgpu_buffer_rsrc_t r, float* dst, int off) {
  if constexpr (VEC)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst), 16, off, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst), 4, off, 0, 0, 0);
}

// Issue the direct-LDS loads of the slice starting at k0 into `stage` (or of
// nothing, when k0 >= K: the resources are then empty and every load writes
// zeros): part PART of PARTS, the wave's A instructions followed by its B
// instructions cut into PARTS consecutive runs.  Completion is waited for
// with vmcnt before the barrier that publishes the stage.
template <class Cfg, bool VA, int PART = 0, int PARTS = 1>
__device__ __forceinline__ void dma_slice(const KernelArgs& p, const DmaLanes<Cfg, VA>& d,
                                          float* stage, int k0, int wave) {
  constexpr Geom g = make_geom(Cfg::tile);
  constexpr int FPL = DmaLanes<Cfg, VA>::FPL, FPL_A = DmaLanes<Cfg, VA>::FPL_A;
  constexpr int NA = dma_ops_a(g, FPL_A), NB = dma_ops_b(g, FPL);
  constexpr int U0 = PART * (NA + NB) / PARTS, U1 = (PART + 1) * (NA + NB) / PARTS;
  const int kr = p.K - k0;
  // Sizes are masked with an opaque all-ones/zero word rather than selected:
  // the compiler turns a select into a branch that duplicates the loads and
  // cuts the loop body into separate scheduling regions.
  int live = __builtin_amdgcn_readfirstlane(~((kr - 1) >> 31));  // -1 when kr > 0
  asm("" : "+s"(live));
  if constexpr (U0 < NA) {
    const auto ra = make_rsrc_exact(d.a_row + k0, (d.a_ext + kr * 4) & live);
#pragma unroll
    for (int j = U0; j < (U1 < NA ? U1 : NA); ++j)
      dma_load<VA && FPL_A == 4>(ra, stage + dma_op(g, wave, j) * 64 * FPL_A, d.a_off[j]);
  }
  if constexpr (U1 > NA) {
    const auto rb = make_rsrc_exact(d.b_col + static_cast<long long>(k0) * p.ldb, d.b_ext & live);
#pragma unroll
    for (int j = (U0 > NA ? U0 : NA) - NA; j < U1 - NA; ++j)
      dma_load<VA>(rb, stage + g.BM * g.BK + dma_op(g, wave, j) * 64 * FPL, d.b_off[j]);
  }
}

// Past the K segment the ring has nothing left to fetch: the last slices'
// loads bring band `band` of this wave's C tile into the caches instead,
// through the freed stage (never read), so the epilogue's first reads of C
// hit.  A band is as many rows as one slice's loads cover in float4s (with
// eight loads per wave, 32 rows of a 64-wide wave tile or 64 rows of a
// 32-wide one); rows past the wave tile are masked.  With beta == 0 the
// resource is empty.
template <class Cfg>
__device__ __forceinline__ void dma_c_band(const KernelArgs& p, float* stage, int crow0, int ccol0,
                                           int band, int wave, int lane) {
  constexpr Geom g = make_geom(Cfg::tile);
  constexpr int NA = dma_ops_a(g, 4), NB = dma_ops_b(g, 4);
  constexpr int LPR = g.WN / 4;            // lanes per wave-tile row
  constexpr int RPO = 64 / LPR;            // rows per load
  static_assert(g.WN % 4 == 0 && 64 % LPR == 0, "wave-tile row width");
  const int rows = min(g.WM, p.M - crow0), cols = min(g.WN, p.N - ccol0);
  int live1 = __builtin_amdgcn_readfirstlane((p.beta != 0.0f && rows > 0 && cols > 0) ? 1 : 0);
  asm("" : "+s"(live1));
  const long long live = live1;
  const auto rc = make_rsrc(p.C + static_cast<long long>(crow0) * p.ldc + ccol0,
                            live * ((static_cast<long long>(rows - 1) * p.ldc + cols) * 4));
  const int ldc = static_cast<int>(p.ldc);
#pragma unroll
  for (int j = 0; j < NA + NB; ++j) {
    const int r = band * (NA + NB) * RPO + j * RPO + lane / LPR, c = (lane % LPR) * 4;
    const int off = (r < rows && c < cols) ? (r * ldc + c) * 4 : kMaskedOffset;
    float* dst = j < NA ? stage + dma_op(g, wave, j) * 256 : stage + g.BM * g.BK + dma_op(g, wave, j - NA) * 256;
    dma_load<true>(rc, dst, off);
  }
}

// Slice 0 (k in [0, r)): the same loads with elements at k >= r masked to
// zero in both operands (so nothing past K, even a non-finite value, meets a
// valid term).  In the float4 variant r % 4 == 0, so a float4 is wholly
// inside or outside.  With A1S the A part loads 4 bytes per lane (the same
// LDS layout), so r need not be a multiple of 4.
template <class Cfg, bool VA, bool A1S = false>
__device__ __forceinline__ void dma_first_slice(const KernelArgs& p, float* stage, int row0,
                                                int col0, int r, int wave, int lane) {
  constexpr Geom g = make_geom(Cfg::tile);
  constexpr int FPL = VA ? 4 : 1;
  constexpr int FPL_A = Cfg::PATH == kPathValu || A1S ? 1 : VA ? 4 : 1;
  const int lda = static_cast<int>(p.lda), ldb = static_cast<int>(p.ldb);
  const int rows = min(g.BM, p.M - row0);
  const auto ra = make_rsrc(p.A + static_cast<long long>(row0) * p.lda,
                            r > 0 ? (static_cast<long long>(rows - 1) * p.lda + r) * 4 : 0);
#pragma unroll
  for (int j = 0; j < dma_ops_a(g, FPL_A); ++j) {
    const MK s = Cfg::PATH == kPathValu ? dma_at_src(g, dma_op(g, wave, j), lane)
                                        : dma_a_src(g, dma_op(g, wave, j), lane, FPL_A);
    dma_load<VA && FPL_A == 4>(ra, stage + dma_op(g, wave, j) * 64 * FPL_A,
                               s.k < r ? (s.m * lda + s.k) * 4 : kMaskedOffset);
  }
  const auto rb = make_rsrc(p.B + col0,
                            r > 0 ? (static_cast<long long>(r - 1) * p.ldb + (p.N - col0)) * 4 : 0);
#pragma unroll
  for (int j = 0; j < dma_ops_b(g, FPL); ++j) {
    const KN s = dma_b_src(g, dma_op(g, wave, j), lane, FPL);
    dma_load<VA>(rb, stage + g.BM * g.BK + dma_op(g, wave, j) * 64 * FPL,
                 s.k < r && s.n < p.N - col0 ? (s.k * ldb + s.n) * 4 : kMaskedOffset);
  }
}

// s_waitcnt immediate that waits for every LDS/scalar-memory operation of
// the wave (lgkmcnt 0, bits 11:8) and leaves vector memory and exports
// unconstrained (vmcnt 63 in bits 3:0 and 15:14, expcnt 7 in bits 6:4).  As a
// builtin, unlike inline asm, the compiler's wait insertion accounts for it.
constexpr int kWaitLgkm0 = 0xc07f;

// Wait until at most N of this wave's vector memory operations are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// Orders the instructions of the scheduling region this call ends: its
// vector memory reads (the slice's direct-to-LDS loads) spread evenly over
// its MFMAs, one after every N_MFMA / N_VM of them.  Left to itself the
// compiler issues the loads in runs of three or four between two MFMAs,
// which stalls the wave's matrix work while they issue.
template <int N_MFMA, int N_VM>
__device__ __forceinline__ void spread_loads() {
  constexpr int kStep = N_MFMA / N_VM;
#pragma unroll
  for (int i = 0; i < N_VM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, kStep, 0);  // kStep MFMAs
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // one vector memory read
  }
}

// Workgroup barrier of the direct-LDS ring: this wave's loads older than its
// N most recent have landed in LDS and its own LDS reads have completed, then
// every wave meets.  __syncthreads() would add a workgroup fence, which also
// drains the N loads meant to stay in flight; the explicit waits are what the
// stage hand-over needs, and the memory clobbers keep the compiler from
// moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Accumulator storage and the inner product, per path.

template <class Cfg, int PATH = Cfg::PATH>
struct Acc;

template <class Cfg>
struct Acc<Cfg, kPathValu> {
  float v[Cfg::WMITER * Cfg::TM * Cfg::WNITER * Cfg::TN];
};

template <class Cfg>
struct Acc<Cfg, kPathMfma32> {
  f32x16 v[Cfg::WMITER][Cfg::WNITER];
};

template <class Cfg>
struct Acc<Cfg, kPathMfma16> {
  f32x4 v[Cfg::WMITER][Cfg::WNITER];
};

template <class Cfg>
__device__ __forceinline__ void acc_zero(Acc<Cfg>& acc) {
  if constexpr (Cfg::PATH == kPathValu) {
#pragma unroll
    for (auto& x : acc.v) x = 0.0f;
  } else {
#pragma unroll
    for (int i = 0; i < Cfg::WMITER; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::WNITER; ++j) acc.v[i][j] = {};
  }
}

// One BK slice of the inner product, reading LDS stage `st`.
template <class Cfg>
__device__ __forceinline__ void inner_product(const float* st, int wr0, int wc0, int lane,
                                              Acc<Cfg>& acc) {
  constexpr Geom g = make_geom(Cfg::tile);
  if constexpr (Cfg::PATH == kPathValu) {
    // Outer product of regM (WMITER*TM values down m) and regN (WNITER*TN
    // values along n) per k, the page's third tiling level, with 128-bit LDS
    // reads.  The fragments of k+1 are read while the FMAs of k run; the
    // scheduling barrier per k-step keeps the compiler from hoisting every
    // read of the slice (which would need BK sets of fragment registers).
    float rm[2][g.WMITER * g.TM], rn[2][g.WNITER * g.TN];
    auto load = [&](int k, int b) {
#pragma unroll
      for (int wm = 0; wm < g.WMITER; ++wm)
#pragma unroll
        for (int i = 0; i < g.TM; i += 4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&st[as_index(g, k, wr0 + valu_m(g, lane, wm, i))]);
#pragma unroll
          for (int q = 0; q < 4; ++q) rm[b][wm * g.TM + i + q] = v[q];
        }
#pragma unroll
      for (int wn = 0; wn < g.WNITER; ++wn)
#pragma unroll
        for (int j = 0; j < g.TN; j += 4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&st[bs_index(g, k, wc0 + valu_n(g, lane, wn, j))]);
#pragma unroll
          for (int q = 0; q < 4; ++q) rn[b][wn * g.TN + j + q] = v[q];
        }
    };
    load(0, 0);
#pragma unroll
    for (int k = 0; k < g.BK; ++k) {
      if (k + 1 < g.BK) load(k + 1, (k + 1) & 1);
      const int b = k & 1;
#pragma unroll
      for (int wm = 0; wm < g.WMITER; ++wm)
#pragma unroll
        for (int i = 0; i < g.TM; ++i)
#pragma unroll
          for (int wn = 0; wn < g.WNITER; ++wn)
#pragma unroll
            for (int j = 0; j < g.TN; ++j) {
              float& a = acc.v[valu_acc_index(g, wm, i, wn, j)];
              a = __builtin_fmaf(rm[b][wm * g.TM + i], rn[b][wn * g.TN + j], a);
            }
      // Keep k-steps apart: LDS reads of later steps may not move above the
      // FMAs of this one (which would need BK sets of fragment registers).
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    constexpr int blk = mfma_blk(g), kstep = mfma_kstep(g);
    const int fr = mfma_frag_row(g, lane), slot = mfma_frag_slot(g, lane);
#pragma unroll
    for (int kk = 0; kk < g.BK; kk += kstep) {
      const int k = kk + slot;
      float a[g.WMITER], b[g.WNITER];
#pragma unroll
      for (int wm = 0; wm < g.WMITER; ++wm) a[wm] = st[as_index(g, k, wr0 + wm * blk + fr)];
#pragma unroll
      for (int wn = 0; wn < g.WNITER; ++wn) b[wn] = st[bs_index(g, k, wc0 + wn * blk + fr)];
#pragma unroll
      for (int wm = 0; wm < g.WMITER; ++wm)
#pragma unroll
        for (int wn = 0; wn < g.WNITER; ++wn) {
          if constexpr (Cfg::PATH == kPathMfma32)
            acc.v[wm][wn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[wm], b[wn], acc.v[wm][wn], 0, 0, 0);
          else
            acc.v[wm][wn] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[wm], b[wn], acc.v[wm][wn], 0, 0, 0);
        }
    }
  }
}

// Fragments of one direct-LDS k-group (8 k for 32x32x2, 16 for 16x16x4):
// per sub-tile row one 128-bit As read (four k of the lane's row, one per
// MFMA), per sub-tile column and MFMA one 32-bit Bs read.  MFMA q takes for
// slot h (lane / blk) the k = group start + 4*h + q.
template <class Cfg>
struct DmaFrag {
  f32x4 a[Cfg::WMITER];
  float b[4][Cfg::WNITER];
};

template <class Cfg>
__device__ __forceinline__ void dma_frag_load(const float* st, int kg, int wr0, int wc0, int lane,
                                              DmaFrag<Cfg>& f) {
  constexpr Geom g = make_geom(Cfg::tile);
  constexpr int blk = mfma_blk(g);
  const int fr = lane % blk, h = lane / blk;
#pragma unroll
  for (int wm = 0; wm < g.WMITER; ++wm)
    f.a[wm] = *reinterpret_cast<const f32x4*>(&st[dma_as_index(g, wr0 + wm * blk + fr, dma_k(g, kg, h, 0))]);
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int wn = 0; wn < g.WNITER; ++wn)
      f.b[q][wn] = st[dma_bs_index(g, dma_k(g, kg, h, q), wc0 + wn * blk + fr)];
}

template <class Cfg>
__device__ __forceinline__ void dma_frag_mfma(const DmaFrag<Cfg>& f, Acc<Cfg>& acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int wm = 0; wm < Cfg::WMITER; ++wm)
#pragma unroll
      for (int wn = 0; wn < Cfg::WNITER; ++wn) {
        if constexpr (Cfg::PATH == kPathMfma32)
          acc.v[wm][wn] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[wm][q], f.b[q][wn], acc.v[wm][wn], 0, 0, 0);
        else
          acc.v[wm][wn] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.a[wm][q], f.b[q][wn], acc.v[wm][wn], 0, 0, 0);
      }
}

// One BK slice of the MFMA inner product over a direct-LDS stage.
template <class Cfg>
__device__ __forceinline__ void inner_product_dma(const float* st, int wr0, int wc0, int lane,
                                                  Acc<Cfg>& acc) {
  constexpr Geom g = make_geom(Cfg::tile);
#pragma unroll
  for (int kg = 0; kg < g.BK / dma_kgroup(g); ++kg) {
    DmaFrag<Cfg> f;
    dma_frag_load<Cfg>(st, kg, wr0, wc0, lane, f);
    dma_frag_mfma<Cfg>(f, acc);
  }
}

// ---- pipelined MFMA loop pieces ---------------------------------------------

template <class Cfg>
struct Frag {
  float a[Cfg::WMITER];
  float b[Cfg::WNITER];
};

// Fragments of the k-step starting at kk (one LDS read per sub-tile row/column).
template <class Cfg>
__device__ __forceinline__ void frag_load(const float* st, int kk, int wr0, int wc0, int lane,
                                          Frag<Cfg>& f) {
  constexpr Geom g = make_geom(Cfg::tile);
  constexpr int blk = mfma_blk(g);
  const int k = kk + mfma_frag_slot(g, lane), fr = mfma_frag_row(g, lane);
#pragma unroll
  for (int wm = 0; wm < g.WMITER; ++wm) f.a[wm] = st[as_index(g, k, wr0 + wm * blk + fr)];
#pragma unroll
  for (int wn = 0; wn < g.WNITER; ++wn) f.b[wn] = st[bs_index(g, k, wc0 + wn * blk + fr)];
}

template <class Cfg>
__device__ __forceinline__ void mfma_step(const Frag<Cfg>& f, Acc<Cfg>& acc) {
#pragma unroll
  for (int wm = 0; wm < Cfg::WMITER; ++wm)
#pragma unroll
    for (int wn = 0; wn < Cfg::WNITER; ++wn) {
      if constexpr (Cfg::PATH == kPathMfma32)
        acc.v[wm][wn] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[wm], f.b[wn], acc.v[wm][wn], 0, 0, 0);
      else
        acc.v[wm][wn] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.a[wm], f.b[wn], acc.v[wm][wn], 0, 0, 0);
    }
}

// K loop with fragment double buffering.  Per slice kt (KS k-steps):
//   issue the global loads of slice kt+1
//   k-steps 0 .. KS-2: read fragments of step s+1, MFMAs of step s;
//                      halfway, write slice kt+1 into the other LDS stage
//   barrier
//   read fragments of step 0 of slice kt+1, then MFMAs of step KS-1 of kt
// The last iteration's extra loads are all masked (k0 >= K reads nothing)
// and its extra LDS writes and reads touch only the unused stage, so the
// loop body has no data-dependent branches.
template <class Cfg, bool VEC>
__device__ __forceinline__ void k_loop_pipelined(const KernelArgs& p, float* lds, int row0,
                                                 int col0, int t, int wr0, int wc0, int lane,
                                                 int kt0, int kt1, Acc<Cfg>& acc) {
  constexpr Geom g = make_geom(Cfg::tile);
  constexpr int kstep = mfma_kstep(g);
  constexpr int KS = g.BK / kstep;
  static_assert(KS % 2 == 0, "pipelined loop needs an even number of k-steps");
  Staged<Cfg> s;
  Frag<Cfg> f[2];
  stage_load<Cfg, VEC>(p, row0, col0, kt0 * g.BK, t, s);
  stage_store<Cfg>(lds, t, s);
  __syncthreads();
  frag_load<Cfg>(lds, 0, wr0, wc0, lane, f[0]);
  for (int kt = kt0; kt < kt1; ++kt) {
    const float* cur = lds + ((kt - kt0) & 1) * g.STAGE;
    float* nxt = lds + ((kt - kt0 + 1) & 1) * g.STAGE;
    stage_load<Cfg, VEC>(p, row0, col0, (kt + 1) * g.BK, t, s);
    // Keep the global loads at the top of the slice: left to itself the
    // scheduler sinks them next to their LDS stores, exposing the full
    // memory latency once per slice.  (The scalar variant's four times more
    // load offsets would not fit the register budget that way.)
    if constexpr (VEC && !(Cfg::OPT & kOptFloatLoads)) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < KS - 1; ++st) {
      frag_load<Cfg>(cur, (st + 1) * kstep, wr0, wc0, lane, f[(st + 1) & 1]);
      mfma_step<Cfg>(f[st & 1], acc);
      if (st == KS / 2 - 1) stage_store<Cfg>(nxt, t, s);
    }
    __syncthreads();
    frag_load<Cfg>(nxt, 0, wr0, wc0, lane, f[0]);
    mfma_step<Cfg>(f[1], acc);
  }
}

// C = alpha*acc + beta*C for in-range elements.  When beta == 0 the old C is
// not read.  `cw` points at C[row0 + wr0][col0 + wc0]; rlim/clim (both >= 1)
// are the rows and columns of the wave tile that lie inside M x N.  One
// buffer resource spans the in-range extent of the wave tile; an element
// outside the window gets kMaskedOffset, so its load reads zero and its store
// is dropped by the hardware's range check (the columns between N and ldc are
// never written).  The body has no per-element branches, and each chunk (one
// MFMA block, or one row of VALU patches) issues all its loads of C before its
// stores, so a wave waits for memory once per chunk rather than once per
// element.
template <class Cfg, bool VEC, class OccCfg = Cfg>
__device__ __forceinline__ void epilogue(float* cw, int ldc, int rlim, int clim, int lane,
                                         float alpha, float beta, const Acc<Cfg>& acc) {
  constexpr Geom g = make_geom(Cfg::tile);
  const auto rc = make_rsrc(cw, (static_cast<long long>(rlim - 1) * ldc + clim) * 4);
  if constexpr (Cfg::PATH == kPathValu) {
    constexpr int V = VEC ? 4 : 1;  // floats per access
    constexpr int PER = g.TM * g.WNITER * g.TN / V;
#pragma unroll
    for (int wm = 0; wm < g.WMITER; ++wm) {
      int off[PER];
#pragma unroll
      for (int i = 0; i < g.TM; ++i)
#pragma unroll
        for (int wn = 0; wn < g.WNITER; ++wn)
#pragma unroll
          for (int j = 0; j < g.TN; j += V) {
            const int r = valu_m(g, lane, wm, i), c = valu_n(g, lane, wn, j);
            // N % 4 == 0 in the float4 variant: a float4 is wholly inside or outside.
            off[(i * g.WNITER * g.TN + wn * g.TN + j) / V] =
                (r < rlim && c < clim) ? (r * ldc + c) * 4 : kMaskedOffset;
          }
      float old[PER][V];
      if (beta != 0.0f) {
#pragma unroll
        for (int x = 0; x < PER; ++x) {
          if constexpr (VEC) {
            const f32x4 o = buffer_load4(rc, off[x]);
#pragma unroll
            for (int q = 0; q < 4; ++q) old[x][q] = o[q];
          } else {
            old[x][0] = buffer_load1(rc, off[x]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < g.TM; ++i)
#pragma unroll
        for (int wn = 0; wn < g.WNITER; ++wn)
#pragma unroll
          for (int j = 0; j < g.TN; j += V) {
            const int x = (i * g.WNITER * g.TN + wn * g.TN + j) / V;
            const int e = valu_acc_index(g, wm, i, wn, j);
            f32x4 v;
#pragma unroll
            for (int q = 0; q < V; ++q) {
              v[q] = alpha * acc.v[e + q];
              if (beta != 0.0f) v[q] = __builtin_fmaf(beta, old[x][q], v[q]);
            }
            if constexpr (VEC) buffer_store4(rc, off[x], v);
            else buffer_store1(rc, off[x], v[0]);
          }
    }
  } else {
    // Sub-tiles in chunks of up to 32 values per lane: every load of a chunk
    // is issued before its first store (a load cannot move above an earlier
    // store to the same buffer), so the C read's memory latency is paid once
    // per chunk rather than once per MFMA block.  Where three or more waves
    // can share a SIMD's registers (the workgroup's own, times the
    // workgroups the LDS or a residency request puts on a CU), one block at
    // a time: the larger chunk spills there, or costs the occupancy.
    constexpr int blk = mfma_blk(g), regs = mfma_regs(g);
    constexpr int kBlocks = g.WMITER * g.WNITER;
    // (OccCfg: the launched tuple, whose threads and LDS set the residency.)
    constexpr int kLdsBlocks = kGfx950.lds_bytes / lds_bytes(OccCfg::tile, kGfx950);
    constexpr int kBlocksPerCu = min_blocks_of(OccCfg::tile) > kLdsBlocks ? min_blocks_of(OccCfg::tile) : kLdsBlocks;
    constexpr int kWavesPerSimd = (OccCfg::NT + 255) / 256 * (kBlocksPerCu > 1 ? kBlocksPerCu : 1);
    constexpr int kValues = kWavesPerSimd >= 3 ? regs : 32;
    constexpr int kChunk = (kValues / regs) < 1 ? 1 : (kValues / regs) > kBlocks ? kBlocks : (kValues / regs);
    const int c_l = mfma_out_col(g, lane);
    if constexpr (kChunk == 1) {
#pragma unroll
      for (int wm = 0; wm < g.WMITER; ++wm)
#pragma unroll
        for (int wn = 0; wn < g.WNITER; ++wn) {
          int off[regs];
          const int c = wn * blk + c_l;
#pragma unroll
          for (int r = 0; r < regs; ++r) {
            const int row = wm * blk + mfma_out_row(g, lane, r);
            off[r] = (row < rlim && c < clim) ? (row * ldc + c) * 4 : kMaskedOffset;
          }
          float old[regs];
          if (beta != 0.0f) {
#pragma unroll
            for (int r = 0; r < regs; ++r) old[r] = buffer_load1(rc, off[r]);
          }
#pragma unroll
          for (int r = 0; r < regs; ++r) {
            float v = alpha * acc.v[wm][wn][r];
            if (beta != 0.0f) v = __builtin_fmaf(beta, old[r], v);
            buffer_store1(rc, off[r], v);
          }
        }
      return;
    }
    auto offset = [&](int b, int r) {
      const int wm = b / g.WNITER, wn = b % g.WNITER;
      const int row = wm * blk + mfma_out_row(g, lane, r), c = wn * blk + c_l;
      return (row < rlim && c < clim) ? (row * ldc + c) * 4 : kMaskedOffset;
    };
#pragma unroll
    for (int b0 = 0; b0 < kBlocks; b0 += kChunk) {
      constexpr int n = kChunk;
      float old[n][regs];
      if (beta != 0.0f) {
#pragma unroll
        for (int b = 0; b < n; ++b)
#pragma unroll
          for (int r = 0; r < regs; ++r)
            if (b0 + b < kBlocks) old[b][r] = buffer_load1(rc, offset(b0 + b, r));
      }
#pragma unroll
      for (int b = 0; b < n; ++b)
#pragma unroll
        for (int r = 0; r < regs; ++r) {
          if (b0 + b >= kBlocks) continue;
          float v = alpha * acc.v[(b0 + b) / g.WNITER][(b0 + b) % g.WNITER][r];
          if (beta != 0.0f) v = __builtin_fmaf(beta, old[b][r], v);
          buffer_store1(rc, offset(b0 + b, r), v);
        }
    }
  }
}

// Split segments: C += alpha * partial with fp32 atomics (C already holds
// beta * C for these tiles).
template <class Cfg>
__device__ __forceinline__ void epilogue_atomic(float* cw, int ldc, int rlim, int clim, int lane,
                                                float alpha, const Acc<Cfg>& acc) {
  constexpr Geom g = make_geom(Cfg::tile);
#pragma unroll
  for (int e = 0; e < g.ACC; ++e) {
    const RC rc = owner(g, 0, lane, e);  // position inside the wave tile (wave 0's origin is 0,0)
    float v;
    if constexpr (Cfg::PATH == kPathValu) {
      v = acc.v[e];
    } else {
      constexpr int regs = mfma_regs(g);
      v = acc.v[(e / regs) / g.WNITER][(e / regs) % g.WNITER][e % regs];
    }
    if (rc.r < rlim && rc.c < clim) unsafeAtomicAdd(cw + rc.r * ldc + rc.c, alpha * v);
  }
}

// Pre-pass for split tiles: C <- beta * C on the tiles at tile-order positions
// [p.tiles_full, tiles_m * tiles_n) (zero when beta == 0, without reading C).
template <int BM, int BN, bool GROUPED>
__global__ void __launch_bounds__(256) sgemm_scale_tiles_kernel(KernelArgs p) {
  const TileRC tc = tile_at(p.tiles_full + static_cast<int>(blockIdx.x), p.tiles_m, p.tiles_n,
                            p.group_m, GROUPED);
  const int row0 = tc.r * BM, col0 = tc.c * BN;
  const int rows = min(BM, p.M - row0), cols = min(BN, p.N - col0);
  float* c = p.C + static_cast<long long>(row0) * p.ldc + col0;
  for (int i = threadIdx.x; i < rows * cols; i += 256) {
    float* e = c + static_cast<long long>(i / cols) * p.ldc + (i % cols);
    *e = p.beta == 0.0f ? 0.0f : p.beta * *e;
  }
}

// The configuration whose geometry the K loop runs with: the tuple itself,
// or for a k-sliced tuple the same tile at half the threads (one wave group).
template <class Cfg, bool KS = (Cfg::OPT & kOptKSlice) != 0>
struct LoopCfg {
  using type = Cfg;
};
template <class Cfg>
struct LoopCfg<Cfg, true> {
  using type = TileCfg<Cfg::BM, Cfg::BN, Cfg::BK, Cfg::WM, Cfg::WN, Cfg::WNITER, Cfg::TM, Cfg::TN,
                       Cfg::NT / 2, Cfg::PATH, Cfg::tile.swz, Cfg::OPT & ~kOptKSlice>;
};

// Accumulator e of a lane (the order epilogue_atomic and owner() use).
template <class Cfg>
__device__ __forceinline__ float acc_get(const Acc<Cfg>& acc, int e) {
  if constexpr (Cfg::PATH == kPathValu) {
    return acc.v[e];
  } else {
    constexpr int regs = Cfg::PATH == kPathMfma32 ? 16 : 4;
    return acc.v[(e / regs) / Cfg::WNITER][(e / regs) % Cfg::WNITER][e % regs];
  }
}
template <class Cfg>
__device__ __forceinline__ void acc_add(Acc<Cfg>& acc, int e, float x) {
  if constexpr (Cfg::PATH == kPathValu) {
    acc.v[e] += x;
  } else {
    constexpr int regs = Cfg::PATH == kPathMfma32 ? 16 : 4;
    acc.v[(e / regs) / Cfg::WNITER][(e / regs) % Cfg::WNITER][e % regs] += x;
  }
}

// The body of the tile kernel (one workgroup, one output tile or K segment).
// HYB (scalar variant of a direct-LDS matrix-core tuple, VEC false): 16-byte
// loads for A in every slice but the first, which loads A 4 bytes per lane,
// and for B in every slice; see sgemm_tile_kernel_hyb.
template <class Cfg, bool VEC, bool HYB = false>
__device__ __forceinline__ void tile_body(const KernelArgs& p) {
  constexpr Geom g = make_geom(Cfg::tile);
  static_assert(tile_legal(Cfg::tile), "illegal tile tuple instantiated");
  constexpr bool kDirect = (Cfg::OPT & kOptDirectLds) != 0;
  static_assert(!HYB || (!VEC && kDirect && Cfg::PATH != kPathValu), "hybrid body: direct-LDS MFMA, scalar variant");
  constexpr bool VA = VEC || HYB;
  constexpr int kStages = kDirect ? stages_of(Cfg::tile) : 2;
  // K-sliced tuples: two wave groups, each with its own LDS ring, run the K
  // loop over the two halves of the slice range with the geometry of half
  // the workgroup (L), and their partial sums are added in LDS afterwards.
  // Every other tuple runs the loop with its own geometry (L = Cfg).
  constexpr bool kKSlice = (Cfg::OPT & kOptKSlice) != 0;
  using L = typename LoopCfg<Cfg>::type;
  constexpr Geom lg = make_geom(L::tile);
  __shared__ __attribute__((aligned(16))) float lds[(kKSlice ? 2 : 1) * kStages * g.STAGE];

  const int t = threadIdx.x;
  const int lane = t & 63;
  // A k-sliced tuple's waves form two groups of kGroupWaves: `half` is the
  // group, `wave` the index within it, and `ro` the offset (floats) of the
  // group's LDS stages.  (All constants of the tuple otherwise; kept as
  // const values selected at compile time, because mutable copies of the
  // wave index or of the LDS pointer change the code the compiler generates
  // for every tuple.)
  constexpr int kGroupWaves = Cfg::NT / (kKSlice ? 128 : 64);
  const int raw_wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int half = kKSlice ? (raw_wave >= kGroupWaves ? 1 : 0) : 0;
  const int wave = kKSlice ? raw_wave - half * kGroupWaves : raw_wave;
  const int ro = kKSlice ? half * kStages * g.STAGE : 0;
  constexpr bool kXcd = (Cfg::OPT & kOptXcdRemap) != 0;
  // Whole tiles first (one workgroup each), then the K segments of the split
  // tiles.
  int pos = blockIdx.x, kt0 = 0, kt1 = p.nk;
  bool split = false;
  if constexpr ((Cfg::OPT & kOptSplitK) != 0) {
    if (pos >= p.tiles_full) {
      const int j = pos - p.tiles_full;
      const int seg = j % p.splits;
      pos = p.tiles_full + j / p.splits;
      kt0 = split_begin(seg, p.splits, p.nk);
      kt1 = split_begin(seg + 1, p.splits, p.nk);
      split = true;
    } else if (kXcd) {
      pos = xcd_position(pos, p.tiles_full);
    }
  } else if (kXcd) {
    pos = xcd_position(pos, p.tiles_m * p.tiles_n);
  }
  const TileRC tc = tile_at(pos, p.tiles_m, p.tiles_n, p.group_m, kXcd);
  const int row0 = tc.r * g.BM;
  const int col0 = tc.c * g.BN;
  // The two groups of a k-sliced tuple run the same number of slices (the
  // second one's last slice lies past K when the count is odd, and loads
  // zeros), so their barriers pair up.
  if constexpr (kKSlice) {
    const int n0 = (kt1 - kt0 + 1) / 2;
    kt0 += half * n0;
    kt1 = kt0 + n0;
  }
  const int wr0 = wave_row0(g, wave), wc0 = wave_col0(g, wave);

  Acc<L> acc;
  acc_zero(acc);

  if constexpr (kDirect) {
    // Direct-LDS staging over a ring of S stages: slice kt+S-1 streams into
    // its stage while slice kt is multiplied.  Before each barrier a wave
    // waits until its loads of slice kt+1 have landed (the S-2 newer slices'
    // loads may stay in flight); the barrier then publishes that stage to
    // every wave and also guarantees that the stage the next iteration loads
    // into (read in this iteration) is no longer read by anyone.  Slices
    // past K load nothing (zeros); past a segment's end they load the next
    // segment's slices, which no one reads.
    constexpr int S = kStages;
    constexpr int kInFlight = (S - 2) * dma_ops_per_slice(L::tile, VA ? 4 : 1);
    const int r = tail_width(p, lg.BK);
    DmaLanes<L, VA> d;
    dma_setup<L, VA>(p, row0, col0, wave, lane, d);
#pragma unroll
    for (int i = 0; i < S - 1; ++i) {
      if (i == 0 && kt0 == 0)
        dma_first_slice<L, VA, HYB>(p, lds + ro, row0, col0, r, wave, lane);
      else
        dma_slice<L, VA>(p, d, lds + ro + i * lg.STAGE, slice_k0(kt0 + i, r, lg.BK), wave);
    }
    ring_barrier<kInFlight>();
    int cur = 0, nxt = S - 1;
    if constexpr ((L::OPT & kOptPipelined) != 0) {
      // Fragments one k-group ahead; the slice's last group is multiplied
      // after the barrier, behind the reads of the next slice's first group
      // (those registers were read before the barrier, so the stage they
      // came from may be refilled).  The loads of slice kt+S go into that
      // freed stage right there, among the last group's MFMAs, so they are
      // spread over matrix work instead of stalling every wave at once, and
      // have nearly S-1 slices to land.  The last iteration reads one group
      // of the stage past the segment, which is never multiplied; the last S
      // slices have no slice left to load, and load either nothing (zeros
      // past K) or, on the tiles named below in the float4 variant, bands of
      // the wave's C tile that the epilogue reads first (dma_c_band).
      constexpr int KG = lg.BK / dma_kgroup(lg);
      // The C prefetch of the last slices pays on the 256x256 tiles of the
      // 32x32 path and on the 128x128 tiles of both paths (one long K loop
      // per tile, C read after it, most of all when C is not in the caches);
      // on 64-row tiles the one-at-a-time tail it needs costs more than it
      // saves.
      constexpr bool kCPrefetch = VA && S == 2 &&
                                  ((L::PATH == kPathMfma32 && lg.BM * lg.BN >= 256 * 256) ||
                                   lg.BM * lg.BN == 128 * 128);
      // MFMAs per k-group and the wave's direct-to-LDS loads per slice:
      // where the group after the barrier has two MFMAs or more per load,
      // the loads are spread over it.
      constexpr int kMf = 4 * lg.WMITER * lg.WNITER;
      constexpr int kVm = dma_ops_a(lg, VA ? 4 : 1) + dma_ops_b(lg, VA ? 4 : 1);
      constexpr bool kSpread = kMf >= 2 * kVm;
      DmaFrag<L> f[2];
      dma_frag_load<L>(lds + ro, 0, wr0, wc0, lane, f[0]);
      dma_slice<L, VA>(p, d, lds + ro + (S - 1) * lg.STAGE, slice_k0(kt0 + S - 1, r, lg.BK), wave);
      // Drain the LDS queue once before the loop: entering it with other
      // LDS work possibly pending makes the compiler wait for every LDS read
      // (lgkmcnt(0)) at the head of each iteration instead of only for the
      // fragments the first MFMAs use.
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      // One slice with stage cs being multiplied.  With two stages the K
      // loop runs two slices per iteration, so each one's stages are
      // constants and its fragment reads take fixed addresses with immediate
      // offsets (no per-slice address arithmetic).  Not in the scalar
      // variant, whose four times as many load offsets leave no registers
      // for the second copy.
      auto slice = [&](int kt, int cs, bool c_band = false) __attribute__((always_inline)) {
        const float* st = lds + ro + cs * lg.STAGE;
        // The scheduling barriers keep each group's reads ahead of the
        // previous group's MFMAs (left alone, the compiler sinks every read
        // to just before its first use and waits for it there).
#pragma unroll
        for (int kg = 0; kg + 1 < KG; ++kg) {
          dma_frag_load<L>(st, kg + 1, wr0, wc0, lane, f[(kg + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          dma_frag_mfma<L>(f[kg & 1], acc);
        }
        ring_barrier<kInFlight>();
        dma_frag_load<L>(lds + ro + (cs + 1 == S ? 0 : cs + 1) * lg.STAGE, 0, wr0, wc0, lane, f[KG & 1]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kCPrefetch) {
          if (c_band)
            dma_c_band<L>(p, lds + ro + cs * lg.STAGE, row0 + wr0, col0 + wc0, kt + S - kt1, wave, lane);
          else
            dma_slice<L, VA>(p, d, lds + ro + cs * lg.STAGE, slice_k0(kt + S, r, lg.BK), wave);
        } else {
          dma_slice<L, VA>(p, d, lds + ro + cs * lg.STAGE, slice_k0(kt + S, r, lg.BK), wave);
        }
        dma_frag_mfma<L>(f[(KG - 1) & 1], acc);
        if constexpr (kSpread) spread_loads<kMf, kVm>();
        if constexpr ((KG & 1) != 0) f[0] = f[1];
      };
      if constexpr (S == 2 && VA && kCPrefetch) {
        int kt = kt0;
        // Pairs while both slices still load real data; the last two or
        // three slices run one at a time, and those past the segment's end
        // prefetch C instead.
        for (; kt + 3 < kt1; kt += 2) {
          slice(kt, 0);
          slice(kt + 1, 1);
        }
        for (; kt < kt1; ++kt) slice(kt, (kt - kt0) & 1, kt + S >= kt1);
      } else if constexpr (S == 2 && VA) {
        int kt = kt0;
        for (; kt + 1 < kt1; kt += 2) {
          slice(kt, 0);
          slice(kt + 1, 1);
        }
        if (kt < kt1) slice(kt, 0);
      } else {
        for (int kt = kt0; kt < kt1; ++kt) {
          slice(kt, cur);
          cur = cur + 1 == S ? 0 : cur + 1;
        }
      }
    } else {
      auto slice = [&](int kt, int cs, int ns) __attribute__((always_inline)) {
        dma_slice<L, VA>(p, d, lds + ro + ns * lg.STAGE, slice_k0(kt + S - 1, r, lg.BK), wave);
        if constexpr (!(L::OPT & kOptFloatLoads)) __builtin_amdgcn_sched_barrier(0);
        // The VALU path reads its transposed A and Bs as register staging
        // lays them out; the MFMA paths read the [m][k] chunk layout.
        if constexpr (L::PATH == kPathValu)
          inner_product<L>(lds + ro + cs * lg.STAGE, wr0, wc0, lane, acc);
        else
          inner_product_dma<L>(lds + ro + cs * lg.STAGE, wr0, wc0, lane, acc);
        ring_barrier<kInFlight>();
      };
      if constexpr (S == 2 && VA) {
        int kt = kt0;
        for (; kt + 1 < kt1; kt += 2) {
          slice(kt, 0, 1);
          slice(kt + 1, 1, 0);
        }
        if (kt < kt1) slice(kt, 0, 1);
      } else {
        for (int kt = kt0; kt < kt1; ++kt) {
          slice(kt, cur, nxt);
          cur = cur + 1 == S ? 0 : cur + 1;
          nxt = nxt + 1 == S ? 0 : nxt + 1;
        }
      }
    }
    // Nothing may still be writing this workgroup's LDS when its waves end.
    if constexpr (kInFlight > 0 || (L::OPT & kOptPipelined) != 0) wait_vmem<0>();
    if constexpr (kKSlice) {
      // The second group's partial sums reach the first through LDS (the
      // rings are free once every wave has passed the barrier): stored
      // lane-contiguous per accumulator, then added in a fixed order, so the
      // result does not depend on timing.
      wait_vmem<0>();
      __syncthreads();
      float* part = lds + wave * (lg.ACC * 64) + lane;
      if (half == 1) {
#pragma unroll
        for (int e = 0; e < lg.ACC; ++e) part[e * 64] = acc_get(acc, e);
      }
      __syncthreads();
      if (half == 1) return;
#pragma unroll
      for (int e = 0; e < lg.ACC; ++e) acc_add(acc, e, part[e * 64]);
    }
  } else if constexpr ((Cfg::OPT & kOptPipelined) != 0) {
    k_loop_pipelined<Cfg, VEC>(p, lds, row0, col0, t, wr0, wc0, lane, kt0, kt1, acc);
  } else {
    Staged<Cfg> s;
    stage_load<Cfg, VEC>(p, row0, col0, kt0 * g.BK, t, s);
    stage_store<Cfg>(lds, t, s);
    __syncthreads();
    // Branch-free body: on the last slice the load reads nothing useful (past
    // K every element is masked; at a segment end it is the next segment's
    // slice) and the store lands in the stage no one reads again.  A branch
    // here would let the compiler sink the whole inner product's arithmetic
    // below it, away from its LDS reads.
    for (int kt = kt0; kt < kt1; ++kt) {
      const float* cur = lds + ((kt - kt0) & 1) * g.STAGE;
      stage_load<Cfg, VEC>(p, row0, col0, (kt + 1) * g.BK, t, s);
      if constexpr (VEC && !(Cfg::OPT & kOptFloatLoads)) __builtin_amdgcn_sched_barrier(0);  // loads stay ahead of the inner product
      inner_product<Cfg>(cur, wr0, wc0, lane, acc);
      stage_store<Cfg>(lds + ((kt - kt0 + 1) & 1) * g.STAGE, t, s);
      __syncthreads();
    }
  }

  const int rlim = min(g.WM, p.M - row0 - wr0);
  const int clim = min(g.WN, p.N - col0 - wc0);
  if (rlim <= 0 || clim <= 0) return;
  float* cw = p.C + static_cast<long long>(row0 + wr0) * p.ldc + (col0 + wc0);
  if constexpr ((Cfg::OPT & kOptSplitK) != 0) {
    if (split) {
      epilogue_atomic<L>(cw, static_cast<int>(p.ldc), rlim, clim, lane, p.alpha, acc);
      return;
    }
  }
  epilogue<L, VEC, Cfg>(cw, static_cast<int>(p.ldc), rlim, clim, lane, p.alpha, p.beta, acc);
}

template <class Cfg, bool VEC>
__global__ void __launch_bounds__(Cfg::NT) sgemm_tile_kernel(KernelArgs p) {
  tile_body<Cfg, VEC>(p);
}

// The same kernel for tuples with a residency request: the register budget is
// capped so that waves_per_eu_of(tile) waves fit each SIMD.  A separate
// template leaves the code generation of every other tuple untouched.
template <class Cfg, bool VEC>
__global__ void __launch_bounds__(Cfg::NT)
    __attribute__((amdgpu_waves_per_eu(waves_per_eu_of(Cfg::tile))))
    sgemm_tile_kernel_occ(KernelArgs p) {
  tile_body<Cfg, VEC>(p);
}

// The scalar variant of a direct-LDS matrix-core tuple (hybrid_scalar_tile):
// 16-byte buffer loads need only 4-byte alignment, and
// every K slice after the first is whole, so A loads 16 bytes per lane in
// those slices whatever K, lda or the operand's alignment; only slice 0,
// when K % 4 != 0, loads A 4 bytes per lane.  B loads 16 bytes per lane
// whatever N: a float4 that starts before column N and crosses it brings the
// row's padding or the next row's first values (zeros past the resource's
// end) into LDS columns at or past N, and those feed only outputs at or past
// column N, which the epilogue never stores; the matrix-core epilogue stores
// element by element.
template <class Cfg>
constexpr bool hybrid_scalar() {
  return hybrid_scalar_tile(Cfg::tile);
}

template <class Cfg>
__global__ void __launch_bounds__(Cfg::NT) sgemm_tile_kernel_hyb(KernelArgs p) {
  tile_body<Cfg, false, true>(p);
}

template <class Cfg>
__global__ void __launch_bounds__(Cfg::NT)
    __attribute__((amdgpu_waves_per_eu(waves_per_eu_of(Cfg::tile))))
    sgemm_tile_kernel_hyb_occ(KernelArgs p) {
  tile_body<Cfg, false, true>(p);
}

template <class Cfg>
const void* hybrid_symbol() {
  if constexpr (min_blocks_of(Cfg::tile) > 0)
    return reinterpret_cast<const void*>(&sgemm_tile_kernel_hyb_occ<Cfg>);
  else
    return reinterpret_cast<const void*>(&sgemm_tile_kernel_hyb<Cfg>);
}

// The kernel of a variant (for the scalar variant of a hybrid tuple, the
// hybrid kernel).
template <class Cfg, bool VEC>
const void* kernel_symbol() {
  if constexpr (!VEC && hybrid_scalar<Cfg>())
    return hybrid_symbol<Cfg>();
  else if constexpr (min_blocks_of(Cfg::tile) > 0)
    return reinterpret_cast<const void*>(&sgemm_tile_kernel_occ<Cfg, VEC>);
  else
    return reinterpret_cast<const void*>(&sgemm_tile_kernel<Cfg, VEC>);
}


// Host-side launcher for one instantiated tuple and variant.
// Tile rows per group of the XCD-aware order: each XCD's share of the tiles
// is made roughly square in elements (rows*BM ~ cols*BN), rounded down to a
// power of two and clamped to the grid.
inline int xcd_group_rows(long long tiles_m, long long tiles_n, int BM, int BN) {
  const double per_xcd = static_cast<double>(tiles_m * tiles_n) / 8.0;
  const double want = per_xcd * BN / BM;
  int g = 1;
  while (static_cast<double>(2 * g) * (2 * g) <= want && 2 * g <= tiles_m) g *= 2;
  return g;
}

// How a launch splits its tiles: the first tiles_full tiles run whole; the
// rest run as `splits` K segments each.  Without the split option, or when
// the tiles fill whole waves of `slots` concurrently resident workgroups (or
// the last wave is at least half full), nothing is split.
struct SplitPlan {
  int tiles_full, splits;
};

inline SplitPlan split_plan(long long tiles, int nk, long long slots, bool enabled) {
  if (!enabled || slots <= 0 || nk < 2) return SplitPlan{static_cast<int>(tiles), 1};
  const long long tail = tiles % slots;
  if (tail == 0 || 2 * tail > slots) return SplitPlan{static_cast<int>(tiles), 1};
  long long s = slots / tail;
  if (s > nk) s = nk;
  if (s < 2) return SplitPlan{static_cast<int>(tiles), 1};
  return SplitPlan{static_cast<int>(tiles - tail), static_cast<int>(s)};
}

// `slots`: workgroups of this kernel that fit on the device at once.
template <class Cfg, bool VEC>
hipError_t launch_tile(const KernelArgs& a, hipStream_t stream, long long slots) {
  KernelArgs k = a;
  const long long tiles_m = (a.M + Cfg::BM - 1) / Cfg::BM;
  const long long tiles_n = (a.N + Cfg::BN - 1) / Cfg::BN;
  if (tiles_m * tiles_n > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  k.tiles_m = static_cast<int>(tiles_m);
  k.tiles_n = static_cast<int>(tiles_n);
  k.group_m = xcd_group_rows(tiles_m, tiles_n, Cfg::BM, Cfg::BN);
  k.nk = (a.K + Cfg::BK - 1) / Cfg::BK;
  const SplitPlan sp = split_plan(tiles_m * tiles_n, k.nk, slots, (Cfg::OPT & kOptSplitK) != 0);
  k.tiles_full = sp.tiles_full;
  k.splits = sp.splits;
  void* args[] = {&k};
  const long long tail = tiles_m * tiles_n - sp.tiles_full;
  if (sp.splits > 1 && a.beta != 1.0f) {
    constexpr bool kGrouped = (Cfg::OPT & kOptXcdRemap) != 0;
    const hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void*>(&sgemm_scale_tiles_kernel<Cfg::BM, Cfg::BN, kGrouped>),
        dim3(static_cast<unsigned>(tail)), dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  const long long grid = sp.tiles_full + tail * sp.splits;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  return hipLaunchKernel(kernel_symbol<Cfg, VEC>(), dim3(static_cast<unsigned>(grid)),
                         dim3(Cfg::NT), args, 0, stream);
}

}  // namespace fp32gemm
