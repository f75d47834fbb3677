// tile_maps.hpp -- every index map the SGEMM kernels use, as constexpr
// functions of a Geom (the tuple plus its derived constants).
//
// The kernels call these with a constexpr Geom, so they fold to constants;
// the host simulator calls the very same functions with runtime Geoms and
// checks, for every tuple, that outputs are owned exactly once, that the
// staging loops cover each tile exactly once, that every LDS access stays in
// its stage and is vector-aligned, and that each lane's fragment reads return
// the (row, k) and (k, col) elements its accumulators need.
//
// Levels follow "Warp Tiling: A Third Level of Tiling" (section "The Kernel"
// and its "Mechanics" list): block tile -> warp (here: wave64) tile ->
// WMITER x WNITER interleaved sub-tiles -> lane patch.
//
// LDS layout.  As holds the A tile transposed, As[k][m] (the page "Vectorized
// Memory Access: 128-bit Loads and Stores", section "Why As Has To Be
// Transposed"), so a lane's consecutive m values sit next to each other.
// Bs holds Bs[k][n] unchanged.  Rows are XOR-swizzled instead of padded.
// With a row stride that is a multiple of the bank count, the transposed
// store of a float4 of A puts every lane of one store phase into the bank
// given by its row m alone -- the conflict that page's section "What Could Be
// Improved" derives, and that grows with BK.  The swizzle, built for a bank
// count NB (the tuple's swz, 32 or 64), XORs m with
//   (k/4 mod KQ) * (NB/KQ)      so the KQ = BK/4 k-groups of one store phase
//                               land on disjoint bank ranges, and
//   a k-parity term (swz_rows)  so the consecutive k-rows that one MFMA
//                               fragment read spreads over its lanes (2 rows
//                               for 32x32x2, 4 for 16x16x4) land on disjoint
//                               bank groups.
// Both terms are multiples of 4 below NB, so aligned float4 groups stay
// contiguous and every row keeps its NB-aligned blocks; Bs gets the second
// term only (its store is a plain row-contiguous float4).
#pragma once

#include "tile_config.hpp"

#if defined(__HIPCC__)
#define FG_HD __host__ __device__
#else
#define FG_HD
#endif

namespace fp32gemm {

struct Geom {
  int BM, BN, BK, WM, WN, WNITER, TM, TN, NT, path, swz, opt;
  int wave, WMITER, WSUBM, WSUBN, WAVES_N, KQ, NQ, ROWS_A, PASSES_A, ROWS_B, PASSES_B;
  int SA, SB, STAGE, ACC;
};

constexpr Geom make_geom(const Tile& t) {
  Geom g{};
  g.BM = t.BM; g.BN = t.BN; g.BK = t.BK; g.WM = t.WM; g.WN = t.WN; g.WNITER = t.WNITER;
  g.TM = t.TM; g.TN = t.TN; g.NT = t.NT; g.path = t.path; g.swz = t.swz; g.opt = t.opt;
  g.wave = 64;
  g.WMITER = wmiter_of(t, 64);
  g.WSUBM = t.WM / g.WMITER;
  g.WSUBN = t.WN / t.WNITER;
  g.WAVES_N = t.BN / t.WN;
  g.KQ = t.BK / 4;
  g.NQ = t.BN / 4;
  g.ROWS_A = t.NT / g.KQ;
  g.PASSES_A = t.BM / g.ROWS_A;
  g.ROWS_B = t.NT / g.NQ;
  g.PASSES_B = t.BK / g.ROWS_B;
  g.SA = lds_stride_a(t);
  g.SB = lds_stride_b(t);
  g.STAGE = lds_floats_per_stage(t);
  g.ACC = acc_per_lane(t, 64);
  return g;
}

// ---- staging: global -> registers -> LDS --------------------------------
// Pass p of thread t loads the float4 A[m][4*kq .. 4*kq+3] of the BM x BK
// block: consecutive threads walk k first, so a row's BK floats are read by
// KQ neighbouring lanes (coalesced along A's contiguous dimension).
FG_HD constexpr int stage_a_row(const Geom& g, int t, int p) { return t / g.KQ + p * g.ROWS_A; }
FG_HD constexpr int stage_a_kq(const Geom& g, int t) { return t % g.KQ; }
// Pass p of thread t loads the float4 B[k][4*nq .. 4*nq+3] of the BK x BN block.
FG_HD constexpr int stage_b_row(const Geom& g, int t, int p) { return t / g.NQ + p * g.ROWS_B; }
FG_HD constexpr int stage_b_nq(const Geom& g, int t) { return t % g.NQ; }

// ---- LDS addresses (floats, relative to one stage) ------------------------
FG_HD constexpr int swz_rows(const Geom& g, int k) {
  // 32 banks: consecutive k-rows differ in bit 4.  64 banks: k-row pairs
  // differ in bit 5 (the two slots of a 32x32x2 fragment read fill both
  // 32-bank halves) and bit 4 separates the pairs (four distinct 16-bank
  // groups for the four slots of a 16x16x4 read).
  return g.swz == 32 ? ((k & 1) << 4) : g.swz == 64 ? (((k & 1) << 5) | ((k & 2) << 3)) : 0;
}
FG_HD constexpr int swz_a(const Geom& g, int k) {
  return g.swz == 0 ? 0 : ((((k >> 2) % g.KQ) * (g.swz / g.KQ)) ^ swz_rows(g, k));
}
FG_HD constexpr int swz_b(const Geom& g, int k) { return swz_rows(g, k); }
FG_HD constexpr int as_index(const Geom& g, int k, int m) { return k * g.SA + (m ^ swz_a(g, k)); }
FG_HD constexpr int bs_index(const Geom& g, int k, int n) {
  return g.BK * g.SA + k * g.SB + (n ^ swz_b(g, k));
}

// ---- direct-LDS staging (MFMA paths) -------------------------------------
// A buffer load that writes LDS places lane l's data at the instruction's LDS
// base + (bytes per lane)*l: each wave instruction fills 64*FPL consecutive
// floats, FPL = 4 for the float4 variant (16-byte loads) and 1 for the scalar
// variant (4-byte loads), and only the global source is chosen per lane.  A
// float4 of A is four k of one row, so this layout keeps As as [m][k]: row m
// holds KQ = BK/4 16-byte chunks, chunk kq stored at chunk position
// kq ^ dma_sw(m).  The fragment read is 128 bits (four k of one row per
// lane); the LDS serves such a read in phases of 8 lanes (32 banks) or 16
// lanes (64 banks), and the swizzle makes the rows a phase touches fall on
// distinct bank groups under both models: with r32 and r64 rows sharing one
// 128-byte or 256-byte bank sweep, it combines the row index divided by each
// (a Gray-code-like XOR, so one term's repeats are the other's distinct
// values).  It repeats every 16 rows.  Bs stays [k][n] with the swz_b chunk
// swizzle.
FG_HD constexpr int dma_sw(const Geom& g, int m) {
  const int r32 = g.KQ >= 8 ? 1 : 8 / g.KQ;
  const int r64 = g.KQ >= 16 ? 1 : 16 / g.KQ;
  const int v = r32 == r64 ? m / r32 : (m / r32) ^ (m / r64);
  return v & (g.KQ - 1);
}
FG_HD constexpr int dma_as_index(const Geom& g, int m, int k) {
  return m * g.BK + 4 * ((k >> 2) ^ dma_sw(g, m)) + (k & 3);
}
// Direct-LDS instructions per wave and slice (A, B) for FPL floats per lane,
// and the workgroup-wide instruction index of a wave's j-th one.
FG_HD constexpr int dma_ops_a(const Geom& g, int fpl) { return g.BM * g.BK / (fpl * g.NT); }
FG_HD constexpr int dma_ops_b(const Geom& g, int fpl) { return g.BK * g.BN / (fpl * g.NT); }
FG_HD constexpr int dma_op(const Geom& g, int w, int j) { return j * (g.NT / 64) + w; }
// Source of lane l in A instruction i: row m and first column k of the FPL
// elements it fetches (they land at float i*64*FPL + FPL*l of the A stage).
struct MK { int m, k; };
FG_HD constexpr MK dma_a_src(const Geom& g, int i, int l, int fpl) {
  const int f = (i * 64 + l) * fpl;
  const int m = f / g.BK, kk = f % g.BK;
  return MK{m, (((kk >> 2) ^ dma_sw(g, m)) << 2) | (kk & 3)};
}
// Bs keeps [k][n] with a column XOR per k-row.  A 32x32x2 fragment read puts
// rows k and k+4 in different 32-lane halves, so the register-staged swz_b
// serves; a 16x16x4 read has four 16-lane slots on rows k, k+4, k+8, k+12,
// which the XOR (k/4 mod 2)*16 (32 banks) or (k/4 mod 4)*16 (64 banks) puts
// on disjoint bank groups.
FG_HD constexpr int dma_swz_b(const Geom& g, int k) {
  return g.path != kPathMfma16 ? swz_b(g, k)
         : g.swz == 0          ? 0
                               : ((k >> 2) & (g.swz == 64 ? 3 : 1)) << 4;
}
FG_HD constexpr int dma_bs_index(const Geom& g, int k, int n) {
  return g.BK * g.SA + k * g.SB + (n ^ dma_swz_b(g, k));
}
// Source of lane l in B instruction i: k-row and first column (LDS float
// BK*BM + i*64*FPL + FPL*l of the stage).
struct KN { int k, n; };
FG_HD constexpr KN dma_b_src(const Geom& g, int i, int l, int fpl) {
  const int f = (i * 64 + l) * fpl;
  const int k = f / g.BN;
  return KN{k, (f % g.BN) ^ dma_swz_b(g, k)};
}
// Direct-LDS staging of A on the VALU path: the inner product reads A
// transposed, As[k][m] (as_index), so these loads move 4 bytes per lane, in
// both variants.  Lane l of A instruction i lands at float i*64 + l of the A
// stage: k-row k = (i*64 + l) / SA at position j = (i*64 + l) % SA, which
// as_index assigns to row m = j ^ swz_a(k).  The swizzle only flips bits
// below 64 and BM is a multiple of 64, so an instruction's 64 floats stay in
// one k-row and the lanes fetch a permutation of 64 consecutive rows at one
// k.
FG_HD constexpr MK dma_at_src(const Geom& g, int i, int l) {
  const int w = i * 64 + l;
  const int k = w / g.SA;
  return MK{(w % g.SA) ^ swz_a(g, k), k};
}

// Fragments: an MFMA block of blk x blk outputs takes, per lane, one A and one
// B value for each of its slots (2 for 32x32x2, 4 for 16x16x4; slot h =
// lane / blk).  The slice's k run in groups of 4*slots; within group kg,
// MFMA q takes for slot h the k = 4*slots*kg + 4*h + q, so one 128-bit read
// of As (chunk slots*kg + h of the lane's row) feeds four MFMAs.
FG_HD constexpr int dma_slots(const Geom& g) { return g.path == kPathMfma16 ? 4 : 2; }
FG_HD constexpr int dma_kgroup(const Geom& g) { return 4 * dma_slots(g); }
FG_HD constexpr int dma_k(const Geom& g, int kg, int h, int q) {
  return dma_kgroup(g) * kg + 4 * h + q;
}

// ---- waves inside the block tile -----------------------------------------
FG_HD constexpr int wave_row0(const Geom& g, int w) { return (w / g.WAVES_N) * g.WM; }
FG_HD constexpr int wave_col0(const Geom& g, int w) { return (w % g.WAVES_N) * g.WN; }

// ---- VALU path: lanes inside one WSUBM x WSUBN sub-tile ---------------------
// The 64 lanes form a (WSUBM/TM) x (WSUBN/TN) grid of TM x TN patches.
FG_HD constexpr int valu_lane_row(const Geom& g, int l) { return l / (g.WSUBN / g.TN); }
FG_HD constexpr int valu_lane_col(const Geom& g, int l) { return l % (g.WSUBN / g.TN); }
// Row (within the wave tile) of regM entry wm*TM + i, and column of regN entry wn*TN + j.
FG_HD constexpr int valu_m(const Geom& g, int l, int wm, int i) {
  return wm * g.WSUBM + valu_lane_row(g, l) * g.TM + i;
}
FG_HD constexpr int valu_n(const Geom& g, int l, int wn, int j) {
  return wn * g.WSUBN + valu_lane_col(g, l) * g.TN + j;
}
// Accumulator e = (wm*TM + i) * (WNITER*TN) + wn*TN + j.
FG_HD constexpr int valu_acc_index(const Geom& g, int wm, int i, int wn, int j) {
  return (wm * g.TM + i) * (g.WNITER * g.TN) + wn * g.TN + j;
}

// ---- MFMA paths ------------------------------------------------------------
// v_mfma_f32_32x32x2_f32: lane l supplies A[i = l%32][s = l/32] and
// B[s = l/32][j = l%32]; accumulator register r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
// v_mfma_f32_16x16x4_f32: lane l supplies A[l%16][l/16] and B[l/16][l%16];
// register r of lane l is D[4*(l/16) + r][l%16].
// Slot s of the k-step starting at kk reads k-row kk + s.
FG_HD constexpr int mfma_blk(const Geom& g) { return g.path == kPathMfma32 ? 32 : 16; }
FG_HD constexpr int mfma_kstep(const Geom& g) { return g.path == kPathMfma32 ? 2 : 4; }
FG_HD constexpr int mfma_regs(const Geom& g) { return g.path == kPathMfma32 ? 16 : 4; }
FG_HD constexpr int mfma_frag_row(const Geom& g, int l) { return l % mfma_blk(g); }
FG_HD constexpr int mfma_frag_slot(const Geom& g, int l) { return l / mfma_blk(g); }
FG_HD constexpr int mfma_out_row(const Geom& g, int l, int r) {
  return g.path == kPathMfma32 ? 8 * (r / 4) + 4 * (l / 32) + (r % 4) : 4 * (l / 16) + r;
}
FG_HD constexpr int mfma_out_col(const Geom& g, int l) { return l % mfma_blk(g); }

// ---- workgroup -> output tile ----------------------------------------------
// Tiles are visited in a "tile order": plain row-major, or (XCD-aware option)
// a grouped raster with group_m tile rows per group, walked column by column
// inside a group.  Workgroup ids map to positions in that order: directly, or
// (XCD-aware) so that the ids the hardware hands to one of the 8 XCDs (id % 8
// equal) get one contiguous run of positions, i.e. one compact block of tiles
// whose A row panels and B column panels that XCD's L2 shares.  Every map
// here is a bijection.
struct TileRC { int r, c; };

FG_HD constexpr TileRC tile_at(int pos, int tiles_m, int tiles_n, int group_m, bool grouped) {
  if (!grouped) return TileRC{pos / tiles_n, pos % tiles_n};
  const int per_group = group_m * tiles_n;
  const int grp = pos / per_group;
  const int first = grp * group_m;
  const int gh = (tiles_m - first) < group_m ? (tiles_m - first) : group_m;
  const int within = pos - grp * per_group;
  return TileRC{first + within % gh, within / gh};
}

// Workgroup id in [0, count) -> position in [0, count): XCD x = id % 8 gets
// the x-th contiguous run.
FG_HD constexpr int xcd_position(int id, int count) {
  const int q = count / 8, rem = count % 8;
  const int x = id % 8, local = id / 8;
  return x * q + (x < rem ? x : rem) + local;
}

FG_HD constexpr TileRC tile_of(int id, int tiles_m, int tiles_n, int group_m, bool xcd) {
  return xcd ? tile_at(xcd_position(id, tiles_m * tiles_n), tiles_m, tiles_n, group_m, true)
             : tile_at(id, tiles_m, tiles_n, group_m, false);
}

// K-slice range [first, last) of segment s when a tile's nk slices are split
// into S segments; the segments partition [0, nk) for any 1 <= S <= nk.
FG_HD constexpr int split_begin(int s, int S, int nk) {
  return static_cast<int>((static_cast<long long>(s) * nk) / S);
}

// ---- output ownership (row, col within the block tile) ---------------------
// Accumulator e of lane l in wave w.
struct RC { int r, c; };
FG_HD constexpr RC owner(const Geom& g, int w, int l, int e) {
  if (g.path == kPathValu) {
    const int row_in = e / (g.WNITER * g.TN);  // wm*TM + i
    const int col_in = e % (g.WNITER * g.TN);  // wn*TN + j
    const int wm = row_in / g.TM, i = row_in % g.TM;
    const int wn = col_in / g.TN, j = col_in % g.TN;
    return RC{wave_row0(g, w) + valu_m(g, l, wm, i), wave_col0(g, w) + valu_n(g, l, wn, j)};
  }
  const int regs = mfma_regs(g), blk = mfma_blk(g);
  const int sub = e / regs, r = e % regs;
  const int wm = sub / g.WNITER, wn = sub % g.WNITER;
  return RC{wave_row0(g, w) + wm * blk + mfma_out_row(g, l, r),
            wave_col0(g, w) + wn * blk + mfma_out_col(g, l)};
}

}  // namespace fp32gemm
