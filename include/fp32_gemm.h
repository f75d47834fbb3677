/*
 * fp32_gemm.h -- C ABI of libfp32_gemm_amd.so, single-precision GEMM on one
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the one every page of the SGEMM series states
 * ("Shared Memory Tiling", kernel listing and epilogue; "Vectorized Memory
 * Access: 128-bit Loads and Stores", section "The Kernel"; "Warp Tiling: A
 * Third Level of Tiling", section "The Kernel"):
 *
 *     C[i,j] <- alpha * sum_{k<K} A[i,k] * B[k,j] + beta * C[i,j]
 *
 * for 0 <= i < M, 0 <= j < N, with row-major matrices addressed through
 * leading dimensions (in elements): X[r,c] = X_ptr[r*ldX + c].  The pages use
 * the tight strides K, N, N; lda/ldb/ldc generalise them.  The sum is
 * accumulated in fp32 in an order the tiling chooses (fp32 MFMA or fp32 FMA,
 * round-to-nearest-even); results agree with the exact sum to
 * max|C - C_exact| / (K * max|A| * max|B|) <= 1e-6.
 *
 * Memory: A, B and C are DEVICE pointers owned by the caller (for example the
 * data pointers of float32 torch tensors on the same GPU).  A and B are only
 * read, C is read (unless beta == 0) and written.  Only the M x N window
 * {C[i*ldc + j] : i < M, j < N} is written; every other byte of C's
 * allocation, including padding columns j >= N, is left untouched.  No byte of
 * A outside its M x K window or of B outside its K x N window is read.  The
 * library allocates nothing per call and keeps no pointer after returning.
 * C must not overlap A or B.
 *
 * Asynchrony: the computation is enqueued on a HIP stream (the default
 * stream for sgemm(), the caller's for sgemm_ex()); buffers must stay alive
 * until the stream passes the call.  Results are visible after a stream
 * synchronisation.  The entry points are thread-safe (no mutable global state
 * besides per-device capability and occupancy caches).  A call may be recorded
 * into a stream capture (HIP graph): it enqueues only kernel launches (two for
 * a split-K configuration: a beta pre-pass and the GEMM), no memset or copy;
 * make one uncaptured call with the same configuration on the device first, so
 * the caches are filled outside the capture.
 *
 * Errors: validation happens before anything is enqueued and never launches.
 * A negative status -i names the i-th argument (1-based) as illegal, BLAS
 * style; positive statuses are run-time conditions (SGEMM_ERR_*).
 */
#ifndef FP32_GEMM_H
#define FP32_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes --------------------------------------------------------- */
#define SGEMM_OK 0
/* -1 M < 0; -2 N < 0; -3 K < 0; -5 A is NULL with M,K > 0; -6 lda < max(1,K);
 * -7 B is NULL with K,N > 0; -8 ldb < max(1,N); -10 C is NULL with M,N > 0;
 * -11 ldc < max(1,N). */
#define SGEMM_ERR_NO_DEVICE 1   /* no current HIP device, or it is not gfx950 */
#define SGEMM_ERR_BAD_CONFIG 2  /* cfg_id is not a compiled configuration */
#define SGEMM_ERR_OVERLAP 3     /* C's M x N extent overlaps A's or B's extent */
#define SGEMM_ERR_LAUNCH 4      /* the kernel launch failed (see sgemm_last_hip_error) */
#define SGEMM_ERR_UNSUPPORTED 5 /* a size beyond the documented limits below */

/* Size limits (SGEMM_ERR_UNSUPPORTED otherwise): M, N, K <= 2^30 and
 * lda, ldb, ldc < 2^21 elements, so that every in-tile byte offset fits the
 * 32-bit offset of a buffer load. */

/* ---- computation ---------------------------------------------------------- */

/* C = alpha*A*B + beta*C on the default (null) stream, with the tuned
 * configuration for this shape.  Argument order and meaning as in the
 * pages' problem statement, plus leading dimensions.
 * Quick returns: M == 0 or N == 0 touches nothing and returns SGEMM_OK;
 * K == 0 computes C = beta*C (empty sum). */
int sgemm(int64_t M, int64_t N, int64_t K, float alpha, const float* A, int64_t lda,
          const float* B, int64_t ldb, float beta, float* C, int64_t ldc);

/* Same computation, enqueued on `stream` (a hipStream_t; NULL = default
 * stream), with configuration `cfg_id` (0 <= cfg_id < sgemm_num_configs()) or
 * the tuned choice when cfg_id < 0.  Operands that are not 16-byte aligned,
 * whose leading dimensions are not multiples of 4, or with K or N not a
 * multiple of 4 run the scalar-load variant of the same configuration.  In
 * that variant the direct-to-LDS matrix-core configurations still load A 16
 * bytes at a time after the first K slice, and B 16 bytes at a time
 * throughout (values that a load brings from past column N reach only
 * outputs past column N, which are never written). */
int sgemm_ex(int64_t M, int64_t N, int64_t K, float alpha, const float* A, int64_t lda,
             const float* B, int64_t ldb, float beta, float* C, int64_t ldc, void* stream,
             int32_t cfg_id);

/* The same computation with the kernel of one rung of the ladder the pages
 * climb, rebuilt for 64-lane waves (reference points, not fast paths except
 * rung 4):
 *   1  shared-memory tiling, one output per lane, 32 x 32 tiles, two
 *      barriers per K step ("Shared Memory Tiling", kernel listing);
 *   2  128 x 128 x 8 tile, 8 x 8 outputs per lane, A transposed in LDS, 128-bit
 *      accesses ("Vectorized Memory Access: 128-bit Loads and Stores");
 *   3  warp tiling, 128 x 64 x 16 tile, 64 x 64 wave tiles, 4 x 4 patches
 *      ("Warp Tiling: A Third Level of Tiling");
 *   4  the tuned dispatch of sgemm_ex (MFMA).
 * Rungs 2-3 run compiled VALU configurations (SGEMM_ERR_BAD_CONFIG if absent);
 * argument rules, status codes and asynchrony as sgemm_ex. */
int sgemm_ladder(int32_t rung, int64_t M, int64_t N, int64_t K, float alpha, const float* A,
                 int64_t lda, const float* B, int64_t ldb, float beta, float* C, int64_t ldc,
                 void* stream);

/* ---- introspection -------------------------------------------------------- */

#define SGEMM_PATH_VALU 0   /* fp32 FMA outer products on the vector ALUs */
#define SGEMM_PATH_MFMA32 1 /* v_mfma_f32_32x32x2_f32 blocks */
#define SGEMM_PATH_MFMA16 2 /* v_mfma_f32_16x16x4_f32 blocks */

/* One compiled tile configuration: the nine-number tuple of "Warp Tiling: A
 * Third Level of Tiling" (section "The Kernel"), the inner-product path, the
 * LDS swizzle's bank model, and derived values. */
typedef struct sgemm_config_t {
  int32_t id;
  int32_t path;
  int32_t BM, BN, BK, WM, WN, WNITER, TM, TN, NT;
  int32_t swz; /* 0 = unswizzled LDS, 32 or 64 = XOR swizzle for that bank count */
  int32_t opt; /* schedule options: bit 0 pipelined MFMA loop (fragments read one k-step,
                  or with bit 4 one k-group, ahead of the MFMAs), bit 1 XCD-aware tile
                  order, bit 2 unpinned global loads, bit 3 split-K for a partly filled
                  last wave (those tiles accumulate with fp32 atomics: not bitwise
                  reproducible), bit 4 direct global-to-LDS loads (both MFMA paths;
                  16-byte loads in the float4 variant, 4-byte loads in the scalar one
                  but for the 16-byte ones described at sgemm_ex),
                  bits 5-6 with bit 4: LDS stages - 2, bits 7-8: workgroups per CU
                  requested - 1 (0 = none), bit 9 k-sliced workgroup (with bit 4:
                  two wave groups of NT/2 threads split the K slices and add their
                  partial sums in LDS, in a fixed order) */
  int32_t WMITER, WSUBM, WSUBN;
  int32_t acc_per_lane;
  int32_t lds_bytes;     /* all LDS stages */
  int32_t vgpr_estimate; /* the checker's estimate; the compiler report is authoritative */
} sgemm_config_t;

int sgemm_num_configs(void);

/* Fills *out for config `id`.  Returns SGEMM_OK or SGEMM_ERR_BAD_CONFIG. */
int sgemm_config_info(int32_t id, sgemm_config_t* out);

/* What sgemm_ex would run for these arguments (no launch, no device needed). */
typedef struct sgemm_plan_t {
  int32_t cfg_id;
  int32_t vector_variant; /* 1 = float4 staging, 0 = scalar staging */
  int64_t grid;           /* workgroups of the GEMM kernel */
  int32_t block;          /* threads per workgroup */
  int32_t tiles_full;     /* output tiles computed whole by one workgroup */
  int32_t splits;         /* K segments of each remaining tile (1 = none) */
  int64_t slots;          /* workgroups of this kernel resident on the current device
                             at once (compute units x occupancy); 0 without a device */
} sgemm_plan_t;

/* Validates like sgemm_ex (same status codes, no device check) and fills
 * *out.  cfg_id < 0 selects the tuned configuration: the exact-shape rule;
 * else, with M, N >= 128 and K >= 32, the tile chosen from the library's
 * table of measured rates (seeded float4-variant shapes on which every
 * table tile was timed; a scalar-variant shape reads them among the tiles
 * whose scalar kernel keeps 16-byte loads): a measured shape's fastest
 * tile, otherwise the tile with the highest sum over the 16 nearest measured
 * shapes in (log2 M, log2 N, log2 K), the K difference weighing 1/2, of
 * exp(-squared distance) * log(rate / that shape's best rate).  Other shapes
 * choose among the rules tuned on shapes of the same variant (all rules if
 * none is): from 2^30 FLOP up and with K >= 256 the largest block tile whose
 * launch keeps at least 85 % of the resident workgroup slots busy (a
 * split-K tuple's split of a partly filled last wave counted; a launch that
 * would split every tile does not count as filling), ties going to the
 * busier launch and then to the nearer rule in (log M, log N, log K); for
 * smaller or shorter-K products, or when no rule fills the device, the
 * nearest rule.
 * Split-K tiles add partial sums with atomics, so their last bits may differ
 * from run to run (within the accuracy bound).  The split decision and the
 * fill check need the device's compute units and occupancy; without a device
 * the fill check is skipped (the nearest rule) and no split is reported; the
 * rate table needs no device. */
int sgemm_plan(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
               int64_t ldb, const float* C, int64_t ldc, int32_t cfg_id, sgemm_plan_t* out);

/* Static string for a status code (never NULL). */
const char* sgemm_status_string(int status);

/* hipError_t of the last failed launch on this thread (0 if none). */
int sgemm_last_hip_error(void);

/* SGEMM_OK if the current HIP device is a gfx950, else SGEMM_ERR_NO_DEVICE. */
int sgemm_device_check(void);

/* Register/LDS/scratch use of a compiled kernel (needs a device).
 * vector_variant selects the float4 kernel (1) or the scalar variant's
 * kernel (0); any other value returns SGEMM_ERR_BAD_CONFIG. */
typedef struct sgemm_kernel_attr_t {
  int32_t num_regs;       /* architectural VGPRs reported by the runtime */
  int32_t scratch_bytes;  /* private (spill) bytes per lane */
  int32_t lds_bytes;      /* static LDS */
  int32_t max_threads;
} sgemm_kernel_attr_t;
int sgemm_kernel_attributes(int32_t id, int32_t vector_variant, sgemm_kernel_attr_t* out);

/* Output tile (row, column in tiles) of each workgroup id for this shape and
 * configuration: fills rows[id], cols[id] for id < min(count, capacity) and
 * returns count = ceil(M/BM) * ceil(N/BN), or -1 for bad arguments.  With
 * the XCD-aware option the order groups each XCD's workgroups into one block
 * of tiles; it is a bijection either way. */
int64_t sgemm_tile_order(int64_t M, int64_t N, int32_t cfg_id, int32_t* rows, int32_t* cols,
                         int64_t capacity);

/* ---- legality checker and index-map simulator ------------------------------ */

/* tuple = {BM, BN, BK, WM, WN, WNITER, TM, TN, NT, path, swz, opt}.
 * target 0 = gfx950 (wave64, 160 KiB LDS, double buffering, register
 * budget); target 1 = the page's own machine model (32-lane warps, 48 KB
 * shared memory, single buffer, <= 128 accumulators), as used by "Autotuning:
 * Searching the Tile-Shape Space".  Returns 0 if legal, else the positive
 * reason code of the first failing guard (see tile_config.hpp), or -1 for a
 * bad target. */
int sgemm_check_tuple(const int32_t tuple[12], int32_t target);

/* Runs the kernels' own index maps on the host for a gfx950-legal tuple and
 * checks: every C element of the block tile owned by exactly one
 * (wave, lane, accumulator); the staging passes cover the A and B slices
 * exactly once with in-bounds, non-colliding, 16-byte aligned LDS addresses;
 * every fragment read returns the element its accumulator needs, and each
 * accumulator sees every k of a slice exactly once.  Also reports the LDS
 * bank-conflict degree of each access class under a banks-wide model
 * (32 or 64 four-byte banks).  For tuples with the direct-LDS option it
 * also checks that layout for both load widths (checks 6-8: the direct
 * loads fill each stage exactly once where the layout expects each element, and the 8-k-group
 * fragment reads feed every accumulator each k once).  Returns 0 when all
 * checks pass, the checker's reason code if the tuple is illegal, or 100+n
 * for failed check n. */
typedef struct sgemm_sim_report_t {
  int32_t failed_check;   /* 0 = all passed */
  int32_t store_a_ways;   /* transposed A store, ds_write_b32 (register-staged layout only; */
  int32_t store_b_ways;   /* B store, ds_write_b128            1 for direct-LDS tuples, which */
  int32_t read_a_ways;    /* fragment reads of As              do not use that layout) */
  int32_t read_b_ways;    /* fragment reads of Bs */
  int32_t dma_read_a_ways; /* direct-LDS option: 128-bit As[m][k] reads (0 without it) */
  int32_t dma_read_b_ways; /* direct-LDS option: Bs reads (0 without it) */
} sgemm_sim_report_t;
int sgemm_simulate_tuple(const int32_t tuple[12], int32_t banks, sgemm_sim_report_t* out);

#ifdef __cplusplus
}
#endif

#endif /* FP32_GEMM_H */
