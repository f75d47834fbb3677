// tile_config.hpp -- the tile tuple, its derived quantities, and the
// compile-time legality checker for the SGEMM kernels.
//
// The tuple is the nine-number parameter list of the warp-tiled kernel on
// "Warp Tiling: A Third Level of Tiling" (section "The Kernel": BM, BN, BK,
// WM, WN, WNITER, TM, TN, NUM_THREADS, with WMITER derived), plus a path tag:
//
//   VALU    : each lane owns WMITER x WNITER patches of TM x TN outputs and
//             forms them as outer products with scalar FMAs.
//   MFMA32  : each WSUBM x WSUBN = 32 x 32 sub-tile is one accumulator block of
//             v_mfma_f32_32x32x2_f32; a lane's share of it is 16 outputs, so the
//             tuple carries TM x TN = 16 x 1.
//   MFMA16  : 16 x 16 sub-tiles of v_mfma_f32_16x16x4_f32; TM x TN = 4 x 1.
//
// The checker restates, for a 64-lane wave, the assumptions the page
// "Autotuning: Searching the Tile-Shape Space" (section "Most Configurations
// Are Not Wrong By A Little") lists for the kernel body: whole waves, whole
// warp tiles, an integral WMITER, exact sub-tile coverage, 4-element vector
// alignment, load loops that tile the staged blocks exactly, single ownership
// of each output, and the shared-memory and accumulator limits.  The guards
// are ordered so that no guard divides by a quantity an earlier guard has not
// already shown to be positive.  On top of those it enforces what the gfx950
// kernels in this library assume: double-buffered LDS within the per-workgroup
// limit, the XOR swizzle's range, the MFMA block shapes and k-step, and an
// estimated register budget.
//
// Everything here is constexpr and free of HIP types, so the same functions
// gate template instantiation (with `if constexpr`), run on the host for the
// tests and the tuner, and feed the index-map simulator.
#pragma once

namespace fp32gemm {

enum Path : int { kPathValu = 0, kPathMfma32 = 1, kPathMfma16 = 2 };

struct Tile {
  int BM, BN, BK, WM, WN, WNITER, TM, TN, NT, path;
  int swz;  // LDS bank count the As/Bs XOR swizzle is built for: 0 (none), 32 or 64
  int opt;  // schedule options, a bit set of kOpt* below
};

// Schedule options.
enum Opt : int {
  // MFMA paths: fragment registers double-buffered across k-steps, the next
  // slice's LDS stores placed mid-slice between MFMAs, and the next slice's
  // first fragments read right after the barrier, ahead of the current
  // slice's last k-step.  With direct-LDS staging the unit is the k-group
  // (one 128-bit A read per sub-tile row): its fragments are read one group
  // ahead, and the slice's last group is multiplied after the barrier, so
  // the matrix cores stay busy while the waves meet.
  kOptPipelined = 1,
  // Workgroup ids remapped so each XCD (the hardware hands consecutive ids to
  // the 8 XCDs in turn) works on one compact block of output tiles.
  kOptXcdRemap = 2,
  // Let the compiler place each slice's global loads (by default they are
  // pinned to the top of the slice in the float4 variant); kept so the two
  // schedules can be compared in one process.
  kOptFloatLoads = 4,
  // Split along K the tiles of a last, partly filled wave of workgroups (or
  // all tiles when they do not fill one wave): their segments add alpha *
  // partial into C with fp32 atomics after a pre-pass has scaled those tiles
  // of C by beta.  Those tiles' sums are therefore not bitwise reproducible
  // from run to run (they stay within the parity bound).
  kOptSplitK = 8,
  // Global -> LDS with buffer loads that write LDS directly (no register
  // round-trip, no ds_write).  MFMA paths: 16-byte loads in the float4
  // variant, 4-byte loads in the scalar variant only for slice 0's A
  // (hybrid_scalar_tile), into an As[m][k] layout
  // whose 16-byte chunks are XOR-swizzled by row; the inner product reads
  // four k of A per 128-bit LDS read.  VALU path: A keeps the transposed,
  // swizzled As[k][m] layout of register staging, filled by 4-byte loads (each
  // lane fetches one row's element at one k), and B is loaded as on the MFMA
  // paths; the inner product is unchanged.
  kOptDirectLds = 16,
  // Direct-LDS option only: a two-bit field giving the LDS stages of the ring,
  // 2 + its value (2, 3 or 4).  With S stages the loads of slice kt+S-1 are
  // issued while slice kt is multiplied, so each slice's loads have S-1
  // slices of compute to land in; the wait before each barrier leaves the
  // S-2 newer slices in flight.
  kOptStagesShift = 5,
  kOptStagesMask = 3 << kOptStagesShift,
  // Residency request (the tuner's occupancy axis): a two-bit field b; b > 0
  // asks the compiler to keep b+1 workgroups resident per CU, i.e. to fit
  // its registers to ceil((b+1) * NT / 256) waves per SIMD -- the role the
  // pages give the second launch-bounds argument.
  kOptOccShift = 7,
  kOptOccMask = 3 << kOptOccShift,
  // K-sliced workgroup (direct-LDS MFMA tuples): NT threads form two groups
  // of NT/2 that each cover the whole block tile with their own LDS ring,
  // over the two halves of the K slices; at the end the second group's
  // accumulators are added to the first's through LDS (a fixed order, no
  // atomics).  It doubles the waves per SIMD of a tile without a second
  // output tile, for shapes with about one tile per compute unit.
  kOptKSlice = 512,
  kOptAll = 1023,
};

constexpr int stages_of(const Tile& t) { return 2 + ((t.opt & kOptStagesMask) >> kOptStagesShift); }

// Tuples whose scalar variant keeps 16-byte loads for A (after the first K
// slice) and for B: the direct-LDS matrix-core tiles (the kernels' hybrid
// scalar body).
constexpr bool hybrid_scalar_tile(const Tile& t) {
  return (t.opt & kOptDirectLds) != 0 && t.path != kPathValu;
}

// Wave groups a k-sliced tuple splits its K loop over (1 otherwise), and the
// tuple one group runs: the same tile at NT / 2 threads without the option.
constexpr int kslices_of(const Tile& t) { return (t.opt & kOptKSlice) ? 2 : 1; }
constexpr Tile half_tile(const Tile& t) {
  return Tile{t.BM, t.BN, t.BK, t.WM, t.WN, t.WNITER, t.TM, t.TN, t.NT / 2, t.path, t.swz,
              t.opt & ~kOptKSlice};
}

// Workgroups per CU the tuple asks for (0 = no request), and the waves per
// SIMD that implies (1 = the compiler's default).
constexpr int min_blocks_of(const Tile& t) {
  return (t.opt & kOptOccMask) ? 1 + ((t.opt & kOptOccMask) >> kOptOccShift) : 0;
}
constexpr int waves_per_eu_of(const Tile& t) {
  return min_blocks_of(t) ? (min_blocks_of(t) * t.NT + 255) / 256 : 1;
}

// Direct-LDS instructions per wave and slice (A plus B) for fpl floats per
// lane (4: float4 variant, 1: scalar variant).  The VALU path loads its
// transposed A 4 bytes per lane in both variants.
constexpr int dma_ops_per_slice(const Tile& t, int fpl) {
  const int fpl_a = t.path == kPathValu ? 1 : fpl;
  return t.BM * t.BK / (fpl_a * t.NT) + t.BK * t.BN / (fpl * t.NT);
}

// Addressing limits.  The kernels form 64-bit tile base addresses but
// in-tile byte offsets in 32 bits: a row index below the block tile height
// (or BK, for B) times a leading dimension, times 4.  Every such offset must
// stay inside one buffer resource, whose record count is at most
// kMaxBufferBytes; the largest accepted leading dimension and the tallest
// block tile are sized together so that it does.
constexpr long long kMaxBufferBytes = 0x7FFFFFF0LL;
constexpr long long kMaxLeadingDim = (1LL << 21) - 1;
constexpr int kMaxTileRows = 256;
static_assert(kMaxTileRows * kMaxLeadingDim * 4 <= kMaxBufferBytes,
              "in-tile offsets of the tallest tile at the largest leading dimension overflow a "
              "buffer resource");

// Machine limits the checker enforces.
struct Target {
  int wave;           // lanes per wave (warp)
  int lds_bytes;      // shared memory available to one workgroup
  int lds_buffers;    // 1 = single-buffered tiles, 2 = double-buffered
  int max_acc;        // accumulators one lane may hold
  int max_arch_vgpr;  // architectural VGPRs per lane (VALU operands)
  int max_vgpr;       // VGPR + AccVGPR per lane
  bool allow_mfma;
  bool gfx950_rules;  // swizzle range, vector reads of As, register estimate
};

// MI355X (gfx950): wave64, 160 KiB LDS per workgroup, double buffering,
// 256 architectural VGPRs + 256 AccVGPRs per lane.
constexpr Target kGfx950{64, 160 * 1024, 2, 256, 256, 512, true, true};

// The page's own machine model: 32-lane warps, 48 KB of static shared memory,
// single-buffered tiles, at most 128 accumulators per thread.
constexpr Target kPageModel{32, 48 * 1024, 1, 128, 1 << 30, 1 << 30, false, false};

// Reason codes, one per guard, in evaluation order.
enum Reason : int {
  kLegal = 0,
  kBadRange = 1,            // a parameter is non-positive, too many threads, or BM or
                            // BK above kMaxTileRows
  kThreadsNotWaves = 2,     // NT is not a whole number of waves
  kBlockNotWarpTiled = 3,   // BM % WM or BN % WN
  kWarpCount = 4,           // warp tiles != waves
  kWmiterFraction = 5,      // WM*WN not divisible by wave*TM*TN*WNITER
  kSubtileSplit = 6,        // WMITER < 1, WM % WMITER or WN % WNITER
  kLaneTile = 7,            // WSUBM % TM or WSUBN % TN
  kSubtileLanes = 8,        // lanes per sub-tile != wave
  kVectorAlign = 9,         // BK, BN, TN (and on gfx950 BM, TM) not multiples of 4
  kLoadStrideA = 10,        // A staging loop does not tile BM x BK exactly
  kLoadStrideB = 11,        // B staging loop does not tile BK x BN exactly
  kOwnership = 12,          // threads x outputs/thread != BM*BN
  kLdsOverflow = 13,        // staged tiles exceed the LDS budget
  kAccOverflow = 14,        // accumulators per lane over the limit
  kMfmaShape = 15,          // MFMA sub-tile / lane tile / k-step mismatch
  kSwizzleRange = 16,       // swizzle needs BM, BN multiples of swz, BK <= swz, BK/4 a power of 2
  kRegisterEstimate = 17,   // estimated registers over the per-lane budget (which shrinks
                            // when one workgroup puts several waves on each SIMD)
  kNoMfmaOnTarget = 18,
  kBadOptions = 19,         // unknown option bits, register-staged pipelining without an even
                            // k-step count, direct-LDS staging without BK in {8, 16, 32, 64}
                            // (16 up for 16x16x4; BM % 64 == 0 on VALU), or a stage ring
                            // without direct-LDS staging,
                            // of 5 stages, or with more loads in flight than vmcnt counts, or a
                            // residency request beyond 8 waves per SIMD or the CU's LDS, or a
                            // k-sliced tuple off the direct-LDS MFMA path or with split-K
  kNumReasons = 20,
};

constexpr int wmiter_of(const Tile& t, int wave) {
  return (t.WM * t.WN) / (wave * t.TM * t.TN * t.WNITER);
}

// Accumulators per lane.
constexpr int acc_per_lane(const Tile& t, int wave) {
  return wmiter_of(t, wave) * t.TM * t.WNITER * t.TN;
}

// Floats per staged A tile row (As is [BK][SA], transposed) and B tile row
// (Bs is [BK][SB]).  The swizzle permutes within a row, so no padding.
constexpr int lds_stride_a(const Tile& t) { return t.BM; }
constexpr int lds_stride_b(const Tile& t) { return t.BN; }

constexpr int lds_floats_per_stage(const Tile& t) {
  return t.BK * lds_stride_a(t) + t.BK * lds_stride_b(t);
}

constexpr int lds_bytes(const Tile& t, const Target& m) {
  const int buffers = (t.opt & kOptDirectLds) && stages_of(t) > m.lds_buffers ? stages_of(t)
                                                                               : m.lds_buffers;
  return kslices_of(t) * buffers * lds_floats_per_stage(t) * 4;
}

// Registers that hold one staged tile between its global load and its LDS
// store (per lane).
constexpr int prefetch_regs(const Tile& t) { return (t.BM * t.BK + t.BK * t.BN) / t.NT; }

// A deliberately rough per-lane register estimate; the compiler's resource
// report is the ground truth and spilling builds are rejected after compile.
constexpr int vgpr_estimate(const Tile& t, int wave) {
  const int wmiter = wmiter_of(t, wave);
  const int fixed = 28;  // addresses, loop state, masks, alpha/beta
  if (t.path == kPathValu) {
    const int frags = 2 * (wmiter * t.TM + t.WNITER * t.TN);
    // Direct-LDS staging holds per-lane load offsets instead of a staged tile.
    const int staging = (t.opt & kOptDirectLds) ? dma_ops_per_slice(t, 4) : prefetch_regs(t);
    return acc_per_lane(t, wave) + frags + staging + fixed;
  }
  // MFMA: fragments are one register per (sub-tile row or column, k-step);
  // accumulators live in AccVGPRs.  Direct-LDS staging holds no staged
  // tile in registers; its fragments are a k-group's four A and four B
  // values per sub-tile row and column, twice when pipelined.
  if (t.opt & kOptDirectLds)  // no staging addresses either
    return ((t.opt & kOptPipelined) ? 8 : 4) * (wmiter + t.WNITER) + fixed - 4;
  const int ksteps = (t.path == kPathMfma32) ? 2 : 1;
  return 2 * ksteps * (wmiter + t.WNITER) + prefetch_regs(t) + fixed;
}

// One workgroup puts ceil(NT / 256) waves on each of a CU's 4 SIMDs, which
// share the SIMD's 512 registers per lane.
constexpr int check_registers(const Tile& t, const Target& m) {
  const int est = vgpr_estimate(t, m.wave);
  const int per_simd = (t.NT / m.wave + 3) / 4;
  const int budget = m.max_vgpr / per_simd;
  if (t.path == kPathValu) {
    if (est > m.max_arch_vgpr || est > budget) return kRegisterEstimate;
  } else {
    const int total = est + acc_per_lane(t, m.wave);
    if (est > m.max_arch_vgpr || total > m.max_vgpr || total > budget) return kRegisterEstimate;
  }
  return kLegal;
}

constexpr int check_tile(const Tile& t, const Target& m);

// A k-sliced tuple is legal when one wave group's tuple is, the option sits
// on a direct-LDS MFMA tuple without the split-K tail (whose segments would
// cross the groups' K ranges), both rings fit the LDS, the second group's
// partial sums (BM x BN floats) fit inside them, and the registers fit with
// both groups' waves on the SIMDs.
constexpr int check_kslice(const Tile& t, const Target& m) {
  if (t.NT <= 0 || t.NT > 1024) return kBadRange;
  if (t.NT % (2 * m.wave) != 0) return kThreadsNotWaves;
  if (t.path == kPathValu || !(t.opt & kOptDirectLds) || (t.opt & kOptSplitK)) return kBadOptions;
  const int h = check_tile(half_tile(t), m);
  if (h != kLegal) return h;
  if (lds_bytes(t, m) > m.lds_bytes || t.BM * t.BN * 4 > lds_bytes(t, m)) return kLdsOverflow;
  if (min_blocks_of(t) > 0 &&
      (waves_per_eu_of(t) > 8 || min_blocks_of(t) * lds_bytes(t, m) > m.lds_bytes))
    return kBadOptions;
  return m.gfx950_rules ? check_registers(t, m) : kLegal;
}

constexpr int check_tile(const Tile& t, const Target& m) {
  if (t.opt & kOptKSlice) return check_kslice(t, m);
  if (t.BM <= 0 || t.BN <= 0 || t.BK <= 0 || t.WM <= 0 || t.WN <= 0 || t.WNITER <= 0 ||
      t.TM <= 0 || t.TN <= 0 || t.NT <= 0 || t.NT > 1024 || t.BM > kMaxTileRows ||
      t.BK > kMaxTileRows)
    return kBadRange;
  if (t.path != kPathValu && !m.allow_mfma) return kNoMfmaOnTarget;
  if ((t.opt & ~kOptAll) != 0) return kBadOptions;

  // Whole waves, tiled evenly by warp tiles.
  if (t.NT % m.wave != 0) return kThreadsNotWaves;
  if (t.BM % t.WM != 0 || t.BN % t.WN != 0) return kBlockNotWarpTiled;
  if ((t.BM / t.WM) * (t.BN / t.WN) != t.NT / m.wave) return kWarpCount;

  // The warp tile splits into whole WMITER x WNITER sub-tiles.
  const int denom = m.wave * t.TM * t.TN * t.WNITER;
  if ((t.WM * t.WN) % denom != 0) return kWmiterFraction;
  const int wmiter = (t.WM * t.WN) / denom;
  if (wmiter < 1 || t.WM % wmiter != 0 || t.WN % t.WNITER != 0) return kSubtileSplit;

  // Each sub-tile is covered by exactly one wave's lanes.
  const int wsubm = t.WM / wmiter, wsubn = t.WN / t.WNITER;
  if (wsubm % t.TM != 0 || wsubn % t.TN != 0) return kLaneTile;
  if ((wsubm / t.TM) * (wsubn / t.TN) != m.wave) return kSubtileLanes;

  // 4-wide vector accesses: global A rows along k, B rows along n, the C
  // epilogue along n; on gfx950 also 128-bit reads of As along m.
  if (t.BK % 4 != 0 || t.BN % 4 != 0) return kVectorAlign;
  if (t.path == kPathValu && t.TN % 4 != 0) return kVectorAlign;
  if (m.gfx950_rules && (t.BM % 4 != 0 || (t.path == kPathValu && t.TM % 4 != 0)))
    return kVectorAlign;

  // Staging loops: every thread loads one float4 per pass; the passes tile
  // the BM x BK block of A and the BK x BN block of B with no remainder.
  if ((t.NT * 4) % t.BK != 0) return kLoadStrideA;
  const int row_stride_a = (t.NT * 4) / t.BK;
  if (row_stride_a < 1 || t.BM % row_stride_a != 0) return kLoadStrideA;
  if (t.NT % (t.BN / 4) != 0) return kLoadStrideB;
  const int row_stride_b = t.NT / (t.BN / 4);
  if (row_stride_b < 1 || t.BK % row_stride_b != 0) return kLoadStrideB;

  // Every output element belongs to exactly one lane.
  if (static_cast<long long>(t.NT) * wmiter * t.TM * t.WNITER * t.TN !=
      static_cast<long long>(t.BM) * t.BN)
    return kOwnership;

  if (t.path == kPathMfma32 || t.path == kPathMfma16) {
    const int blk = (t.path == kPathMfma32) ? 32 : 16;
    const int tm = (t.path == kPathMfma32) ? 16 : 4;
    const int kstep = (t.path == kPathMfma32) ? 2 : 4;
    if (wsubm != blk || wsubn != blk || t.TM != tm || t.TN != 1 || t.BK % kstep != 0)
      return kMfmaShape;
    // The pipelined loop alternates two fragment buffers per k-step and
    // relies on an even number of k-steps per slice.
    if ((t.opt & kOptPipelined) && !(t.opt & kOptDirectLds) && (t.BK / kstep) % 2 != 0)
      return kBadOptions;
  } else if (t.opt & kOptPipelined) {
    return kBadOptions;
  }
  // Direct-LDS staging: on the MFMA paths in their own loop (pipelined by
  // k-group rather than by k-step), with whole k-groups per slice (8 k for
  // 32x32x2, 16 for 16x16x4) and a power-of-two number of 16-byte chunks per
  // As row (the chunk swizzle is an XOR below that count).  On the VALU path
  // A stays transposed and each 4-byte load instruction fills 64 floats of
  // one As row, so BM is a multiple of 64.
  if ((t.opt & kOptDirectLds) &&
      ((t.BK != 8 && t.BK != 16 && t.BK != 32 && t.BK != 64) ||
       (t.path == kPathMfma16 && t.BK < 16) || (t.path == kPathValu && t.BM % 64 != 0)))
    return kBadOptions;
  // The stage ring belongs to the direct-LDS loop; at most 4 stages, and the
  // loads left in flight at each wait fit the 6-bit vmcnt counter.
  if ((t.opt & kOptStagesMask) != 0 &&
      (!(t.opt & kOptDirectLds) || stages_of(t) > 4 || (stages_of(t) - 2) * dma_ops_per_slice(t, 1) > 63))
    return kBadOptions;

  if (m.gfx950_rules) {
    // The As/Bs XOR swizzle flips bits below swz, in steps of at least 4
    // words, so it needs swz-aligned rows and at most swz/4 groups of four
    // k-rows per staged tile.  Direct-LDS MFMA tuples keep As as [m][k] with
    // their own chunk swizzle; for them only the Bs part applies.
    if (t.swz != 0 && t.swz != 32 && t.swz != 64) return kSwizzleRange;
    if (t.swz != 0 && t.BN % t.swz != 0) return kSwizzleRange;
    if (t.swz != 0 && (!(t.opt & kOptDirectLds) || t.path == kPathValu) &&
        (t.BM % t.swz != 0 || t.BK > t.swz || ((t.BK / 4) & (t.BK / 4 - 1)) != 0))
      return kSwizzleRange;
  }

  if (lds_bytes(t, m) > m.lds_bytes) return kLdsOverflow;
  // A residency request must be satisfiable: its waves fit a SIMD (8) and its
  // workgroups' LDS fits the CU.
  if (min_blocks_of(t) > 0 &&
      (waves_per_eu_of(t) > 8 || min_blocks_of(t) * lds_bytes(t, m) > m.lds_bytes))
    return kBadOptions;
  const int acc_limit = (t.path == kPathValu) ? (m.max_acc < 128 ? m.max_acc : 128) : m.max_acc;
  if (acc_per_lane(t, m.wave) > acc_limit) return kAccOverflow;

  if (m.gfx950_rules) return check_registers(t, m);
  return kLegal;
}

constexpr bool tile_legal(const Tile& t) { return check_tile(t, kGfx950) == kLegal; }

// Compile-time view of a legal tuple with its derived constants.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int WNITER_, int TM_, int TN_, int NT_,
          int PATH_, int SWZ_, int OPT_>
struct TileCfg {
  static constexpr Tile tile{BM_, BN_, BK_, WM_, WN_, WNITER_, TM_, TN_, NT_, PATH_, SWZ_, OPT_};
  static constexpr int OPT = OPT_;
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, WNITER = WNITER_;
  static constexpr int TM = TM_, TN = TN_, NT = NT_, PATH = PATH_;
  static constexpr int WAVE = 64;
  static constexpr int WMITER = wmiter_of(tile, WAVE);
  static constexpr int WSUBM = WM / WMITER, WSUBN = WN / WNITER;
  static constexpr int WAVES_N = BN / WN;  // warp tiles across the block tile
  static constexpr int KQ = BK / 4;        // float4 columns in a staged A row
  static constexpr int NQ = BN / 4;        // float4 columns in a staged B row
  static constexpr int ROWS_A = NT / KQ;   // A rows staged per pass
  static constexpr int PASSES_A = BM / ROWS_A;
  static constexpr int ROWS_B = NT / NQ;   // B rows staged per pass
  static constexpr int PASSES_B = BK / ROWS_B;
  static constexpr int SA = lds_stride_a(tile), SB = lds_stride_b(tile);
  static constexpr int STAGE_FLOATS = lds_floats_per_stage(tile);
};

}  // namespace fp32gemm
