"""Operation counts, traffic model and MI355X roofs for SGEMM.

Formulas restated from the pages: the operation count 2*M*N*K ("Warp Tiling:
A Third Level of Tiling", section "Retiring The Roofline"), the global-access
count per output K*(1/BM + 1/BN) and the shared-memory count per output
(section "The Arithmetic, As A Negative Result"; "Vectorized Memory Access:
128-bit Loads and Stores", section "Instructions, Not Bytes").
"""
from __future__ import annotations

# MI355X (gfx950) published peaks.
CUS = 256
CLOCK_HZ = 2.4e9
FP32_FLOP_PER_CLK_PER_CU = 256          # MFMA fp32, or VALU with packed FMA
PEAK_FP32_TFLOPS = CUS * CLOCK_HZ * FP32_FLOP_PER_CLK_PER_CU / 1e12   # 157.3 (matrix and vector)
# Without packed-FP32 instructions one VALU FMA instruction covers one FMA per
# lane: nominally half the published vector peak.  (Register-only probes
# measure the three-operand v_fma_f32 at about 75 TFLOP/s and the two-operand
# v_fmac_f32 at 122.7 TFLOP/s, so the issue rate, not this nominal half, is
# what bounds the VALU path.)
PEAK_FP32_VALU_UNPACKED_TFLOPS = PEAK_FP32_TFLOPS / 2                  # 78.6
PEAK_HBM_GBS = 8000.0


def flops(M, N, K):
    """Multiply-adds counted as two operations; the epilogue is not counted."""
    return 2 * M * N * K


def algorithmic_bytes(M, N, K, beta):
    """Bytes the operation must move at least: read A and B once, write C,
    and read C when beta != 0."""
    b = 4 * (M * K + K * N + M * N)
    if beta != 0:
        b += 4 * M * N
    return b


def gmem_loads_per_output(BM, BN, K):
    """Global loads per output element for a BM x BN block tile."""
    return K * (1.0 / BM + 1.0 / BN)


def requested_bytes(BM, BN, M, N, K):
    """Bytes the block tiles request from the memory system for A and B."""
    return 4 * M * N * gmem_loads_per_output(BM, BN, K)


def lds_loads_per_output(WMITER, TM, WNITER, TN, K):
    """Shared-memory values read per output: per k a lane reads WMITER*TM +
    WNITER*TN values to feed WMITER*TM*WNITER*TN accumulators."""
    return K * (WMITER * TM + WNITER * TN) / (WMITER * TM * WNITER * TN)


def tflops(M, N, K, seconds):
    return flops(M, N, K) / seconds / 1e12
