"""Legality checker, index-map simulator and traffic model (CPU only).

The checker is pinned to the structure numbers the pages print for their own
warp-tiled configuration (tests/golden/page_structure.json), evaluated in the
page's machine model (32-lane warps, 48 KB shared memory); every guard has a
tuple that trips it first; and every configuration compiled into the library
passes the host simulation of the kernels' own index maps.
"""
import json
import os

import pytest

import fp32_gemm_amd as fg
from fp32_gemm_amd import model

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_structure.json")))
VALU, MFMA32, MFMA16 = 0, 1, 2


def page_tuple():
    t = GOLD["warp_tiled_kernel"]["tuple"]
    return (t["BM"], t["BN"], t["BK"], t["WM"], t["WN"], t["WNITER"], t["TM"], t["TN"], t["NT"],
            VALU, 0)


def test_page_tuple_is_legal_in_page_model_with_printed_structure():
    g = GOLD["warp_tiled_kernel"]
    tup = page_tuple()
    assert fg.check_tuple(tup, "page") == 0
    BM, BN, BK, WM, WN, WNITER, TM, TN, NT = tup[:9]
    warp = g["warp"]
    wmiter = (WM * WN) // (warp * TM * TN * WNITER)
    assert wmiter == g["WMITER"]
    assert (WM // wmiter, WN // WNITER) == (g["WSUBM"], g["WSUBN"])
    assert [(WM // wmiter) // TM, (WN // WNITER) // TN] == g["lane_grid"]
    assert warp * TM * TN == g["outputs_per_warp_pass"] and WM * WN == g["warp_tile_outputs"]
    assert NT * 4 // BK == g["row_stride_a"] and BM // g["row_stride_a"] == g["passes_a"]
    assert NT // (BN // 4) == g["row_stride_b"] and BK // g["row_stride_b"] == g["passes_b"]
    assert wmiter * TM * WNITER * TN == g["accumulators"]


def test_page_tuple_needs_reshaping_for_wave64():
    # Four 64x32 warp tiles but only two 64-lane waves in 128 threads.
    assert fg.check_tuple(page_tuple(), "gfx950") == 4
    # Widening the warp tile to 64x64 makes it a legal wave64 tuple.
    t = list(page_tuple()); t[4] = 64; t[10] = 32
    assert fg.check_tuple(tuple(t), "gfx950") == 0
    assert fg.simulate_tuple(tuple(t))["status"] == 0


def test_vectorized_kernel_numbers():
    v = GOLD["vectorized_kernel"]
    assert (v["BM"] * v["BN"]) // (v["TM"] * v["TN"]) == v["threads"]
    assert v["threads"] * 4 == v["tile_elements"] == v["BM"] * v["BK"] == v["BN"] * v["BK"]
    assert v["BK"] // 4 == v["a_float4_columns"] and v["threads"] // (v["BK"] // 4) == v["a_rows"]
    assert v["BN"] // 4 == v["b_float4_columns"] and v["threads"] // (v["BN"] // 4) == v["b_rows"]


# One tuple per guard, each tripping that guard first (gfx950 target).
GUARD_CASES = [
    (1, (0, 64, 16, 64, 64, 2, 4, 4, 64, VALU, 32)),
    (2, (128, 64, 16, 64, 64, 2, 4, 4, 96, VALU, 32)),
    (3, (128, 64, 16, 48, 64, 2, 4, 4, 128, VALU, 32)),
    (4, (128, 64, 16, 64, 32, 2, 4, 4, 128, VALU, 32)),
    (5, (128, 128, 16, 64, 64, 1, 12, 4, 256, VALU, 32)),
    (6, (32, 96, 16, 32, 96, 1, 4, 4, 64, VALU, 32)),
    (7, (128, 96, 12, 128, 96, 1, 12, 8, 64, VALU, 32)),
    (9, (128, 128, 16, 64, 64, 2, 2, 8, 256, VALU, 32)),
    (10, (96, 128, 12, 48, 128, 1, 1, 2, 128, MFMA32, 32)),
    (11, (96, 32, 8, 32, 32, 1, 2, 2, 192, MFMA32, 32)),
    (13, (256, 256, 64, 128, 128, 4, 16, 1, 256, MFMA32, 64)),
    (14, (96, 128, 8, 96, 128, 2, 4, 4, 64, VALU, 32)),
    (15, (128, 128, 16, 64, 64, 4, 16, 1, 256, MFMA32, 32)),
    (16, (96, 128, 16, 96, 64, 2, 16, 1, 128, MFMA32, 64)),
    (17, (128, 128, 32, 64, 128, 1, 16, 4, 128, VALU, 32)),
]


@pytest.mark.parametrize("reason,tup", GUARD_CASES)
def test_each_guard_trips(reason, tup):
    assert fg.check_tuple(tup, "gfx950") == reason


def test_kslice_rules():
    # K-sliced workgroups: legal exactly when one wave group's tuple is, on
    # the direct-LDS MFMA path without split-K, with both groups' LDS rings
    # (and the partial-sum buffer) inside the CU's LDS.
    ks = 512
    base = (64, 64, 64, 32, 32, 1, 16, 1, 512, MFMA32, 32)
    assert fg.check_tuple(base + (16 | ks,), "gfx950") == 0
    assert fg.check_tuple(base[:8] + (256,) + base[9:] + (16,), "gfx950") == 0  # one group's tuple
    assert fg.check_tuple(base + (ks,), "gfx950") == 19            # not direct-LDS
    assert fg.check_tuple(base + (16 | 8 | ks,), "gfx950") == 19   # with split-K
    assert fg.check_tuple((128, 64, 16, 64, 64, 2, 4, 4, 256, VALU, 32, ks), "gfx950") == 19
    assert fg.check_tuple(base[:8] + (384,) + base[9:] + (16 | ks,), "gfx950") == 4  # 3 waves per group
    # 128 x 128 x 64: two rings of two 64 KiB stages exceed 160 KiB.
    assert fg.check_tuple((128, 128, 64, 64, 64, 2, 16, 1, 512, MFMA32, 32, 16 | ks), "gfx950") == 13
    # 256 x 256 x 8: the rings fit, the 256 KiB partial-sum buffer does not.
    assert fg.check_tuple((256, 256, 8, 128, 128, 4, 16, 1, 512, MFMA32, 32, 16 | ks), "gfx950") == 13
    for c in fg.configs():
        if c["opt"] & ks:
            half = c["tuple"][:8] + (c["NT"] // 2,) + c["tuple"][9:11] + (c["opt"] & ~ks,)
            assert fg.check_tuple(half, "gfx950") == 0, c["tuple"]
            assert c["lds_bytes"] >= c["BM"] * c["BN"] * 4


def test_tile_height_limit():
    # In-tile offsets are 32-bit: a block tile taller than 256 rows at the
    # largest leading dimension (2^21 - 1) would leave a buffer resource's
    # range, so the range guard rejects it although every other guard holds.
    tall = (512, 64, 16, 128, 64, 1, 4, 4, 256, VALU, 0)
    assert fg.check_tuple(tall, "gfx950") == 1
    assert fg.check_tuple((256, 64, 16, 128, 64, 1, 4, 4, 128, VALU, 0), "gfx950") != 1
    assert 256 * ((1 << 21) - 1) * 4 <= 0x7FFFFFF0 < 512 * ((1 << 21) - 1) * 4


def test_lane_count_and_ownership_guards_are_implied():
    """Guards 8 (lanes per sub-tile) and 12 (single ownership) cannot trip
    first: once WMITER divides exactly (guards 5-7), the lanes per sub-tile
    are WM*WN/(WMITER*TM*WNITER*TN) = wave, and threads x outputs per thread
    equals BM*BN by the warp count (guard 4).  A random sweep confirms no
    tuple reaches them."""
    import random
    rng = random.Random(7)
    vals = [[32, 64, 96, 128], [32, 64, 96, 128], [8, 12, 16, 32], [16, 32, 48, 64, 96, 128],
            [16, 32, 64, 96, 128], [1, 2, 3, 4], [1, 2, 4, 8, 12, 16], [1, 2, 4, 8],
            [64, 128, 192, 256], [0, 1, 2], [0, 32]]
    seen = set()
    for _ in range(20000):
        seen.add(fg.check_tuple(tuple(rng.choice(v) for v in vals), "gfx950"))
        seen.add(fg.check_tuple(tuple(rng.choice(v) for v in vals), "page"))
    assert 8 not in seen and 12 not in seen
    assert {3, 4, 5, 6, 7, 9, 10, 11} <= seen


def test_page_model_limits():
    # 48 KB of shared memory in the page model, single-buffered.
    big = (256, 256, 32, 64, 64, 2, 4, 4, 512, VALU, 0)
    assert fg.check_tuple(big, "page") == 13
    # The MFMA paths do not exist in the page model.
    assert fg.check_tuple((128, 128, 16, 64, 64, 2, 16, 1, 256, MFMA32, 32), "page") == 18


def test_every_compiled_config_is_legal_and_simulates():
    cfgs = fg.configs()
    assert len(cfgs) > 20
    for c in cfgs:
        assert fg.check_tuple(c["tuple"], "gfx950") == 0, c
        rep = fg.simulate_tuple(c["tuple"], banks=32)
        assert rep["status"] == 0, (c["tuple"], rep)


def test_swizzle_removes_modelled_bank_conflicts():
    base = (256, 256, 16, 128, 128, 4, 16, 1, 256, MFMA32)
    plain = fg.simulate_tuple(base + (0,), banks=32)
    swz = fg.simulate_tuple(base + (32,), banks=32)
    swz64 = fg.simulate_tuple(base + (64,), banks=64)
    assert plain["status"] == swz["status"] == swz64["status"] == 0
    # Unswizzled transposed store at BK = 16: a 32-lane phase covers 8 rows,
    # so each bank serves 4 distinct words.
    assert plain["store_a_ways"] == 4
    assert swz["store_a_ways"] == 1 and swz["read_a_ways"] == 1 and swz["read_b_ways"] == 1
    assert swz64["store_a_ways"] == 1 and swz64["read_a_ways"] == 1 and swz64["read_b_ways"] == 1


def test_bank_conflict_of_unswizzled_transpose_matches_page_derivation():
    k = GOLD["bank_conflict_k7"]
    # BK = 8: 32 lanes cover 16 rows -> 2-way (the page's kernel-7 derivation).
    t8 = (128, 64, 8, 64, 64, 2, 4, 4, 128, VALU, 0)
    assert 32 // (8 // 4) == k["BK8_rows_per_warp"]
    assert fg.simulate_tuple(t8, banks=32)["store_a_ways"] == k["BK8_ways"]
    t16 = (128, 64, 16, 64, 64, 2, 4, 4, 128, VALU, 0)
    assert 32 // (16 // 4) == k["BK16_rows_per_warp"]
    assert fg.simulate_tuple(t16, banks=32)["store_a_ways"] == 32 // k["BK16_rows_per_warp"]


def test_traffic_model_matches_page_numbers():
    t = GOLD["traffic"]
    K = t["K"]
    assert model.gmem_loads_per_output(128, 64, K) == t["gmem_per_output_128x64"]
    assert model.gmem_loads_per_output(128, 128, K) == t["gmem_per_output_128x128"]
    assert round(model.requested_bytes(128, 128, K, K, K) / 1e9, 2) == t["gmem_total_GB_128x128"]
    assert round(model.requested_bytes(128, 64, K, K, K) / 1e9, 2) == t["gmem_total_GB_128x64"]
    assert model.lds_loads_per_output(2, 4, 2, 4, K) == t["smem_loads_per_output"]
    assert model.lds_loads_per_output(1, 8, 1, 8, K) == t["smem_loads_per_output"]
    assert round(model.flops(K, K, K) / 1e9, 2) == t["gflop_4096"]


def test_peak_numbers():
    assert abs(model.PEAK_FP32_TFLOPS - 157.286) < 0.01
    assert abs(model.PEAK_FP32_VALU_UNPACKED_TFLOPS - 78.643) < 0.01


def test_option_guard():
    # Pipelining is an MFMA-loop option and needs an even number of k-steps.
    assert fg.check_tuple((128, 64, 16, 64, 64, 2, 4, 4, 128, VALU, 32, 1)) == 19
    assert fg.check_tuple((128, 128, 4, 128, 64, 4, 4, 1, 128, MFMA16, 0, 1)) == 19
    assert fg.check_tuple((128, 128, 16, 64, 64, 2, 16, 1, 256, MFMA32, 32, 1024)) == 19  # unknown bit
    assert fg.check_tuple((128, 128, 16, 64, 64, 2, 16, 1, 256, MFMA32, 32, 3)) == 0
    # Direct-LDS staging: BK a power of two from 8 to 64 (from 16 for
    # 16x16x4, whose k-group is 16).  Its MFMA pipeline works per k-group, so
    # an odd k-group count (one, here) is fine.  On the VALU path (A loaded
    # transposed, 64 rows per load instruction) BM must be a multiple of 64,
    # and the k-group pipeline does not apply.
    assert fg.check_tuple((128, 128, 16, 64, 64, 2, 16, 1, 256, MFMA32, 32, 16)) == 0
    assert fg.check_tuple((128, 128, 16, 64, 64, 2, 16, 1, 256, MFMA32, 32, 17)) == 0
    assert fg.check_tuple((128, 128, 8, 64, 64, 2, 16, 1, 256, MFMA32, 32, 17)) == 0
    assert fg.check_tuple((128, 128, 16, 64, 64, 4, 4, 1, 256, MFMA16, 32, 16)) == 0
    assert fg.check_tuple((128, 128, 16, 64, 64, 4, 4, 1, 256, MFMA16, 32, 17)) == 0
    assert fg.check_tuple((128, 128, 8, 64, 64, 4, 4, 1, 256, MFMA16, 32, 16)) == 19
    assert fg.check_tuple((128, 64, 16, 64, 64, 2, 4, 4, 128, VALU, 32, 16)) == 0
    assert fg.check_tuple((128, 64, 16, 64, 64, 2, 4, 4, 128, VALU, 32, 17)) == 19
    assert fg.check_tuple((96, 64, 16, 96, 64, 2, 4, 4, 64, VALU, 32, 0)) == 0
    assert fg.check_tuple((96, 64, 16, 96, 64, 2, 4, 4, 64, VALU, 32, 16)) == 19
    assert fg.check_tuple((128, 64, 64, 64, 64, 2, 4, 4, 128, VALU, 32, 16)) == 16  # swizzle range
    assert fg.check_tuple((96, 64, 24, 32, 64, 2, 16, 1, 192, MFMA32, 0, 16)) == 19
    # Stage rings (opt field 32 = 3 stages, 64 = 4): direct-LDS only, at most 4
    # stages, and the LDS budget counts every stage.
    assert fg.check_tuple((128, 128, 16, 64, 64, 2, 16, 1, 256, MFMA32, 32, 16 | 64)) == 0
    assert fg.check_tuple((128, 128, 16, 64, 64, 2, 16, 1, 256, MFMA32, 32, 64)) == 19
    assert fg.check_tuple((128, 128, 16, 64, 64, 2, 16, 1, 256, MFMA32, 32, 16 | 96)) == 19
    assert fg.check_tuple((256, 256, 32, 64, 128, 4, 16, 1, 512, MFMA32, 32, 16)) == 0
    assert fg.check_tuple((256, 256, 32, 64, 128, 4, 16, 1, 512, MFMA32, 32, 16 | 32)) == 13
    assert fg.check_tuple((256, 256, 16, 64, 128, 4, 16, 1, 512, MFMA32, 32, 16 | 64)) == 0
    # Residency requests (opt field 128 * b: b + 1 workgroups per CU) must fit
    # 8 waves per SIMD and the CU's LDS.
    assert fg.check_tuple((128, 128, 16, 32, 64, 2, 16, 1, 512, MFMA32, 32, 16 | 3 << 7)) == 0
    assert fg.check_tuple((128, 128, 32, 32, 32, 1, 16, 1, 1024, MFMA32, 32, 1 << 7)) == 0
    assert fg.check_tuple((128, 128, 32, 32, 32, 1, 16, 1, 1024, MFMA32, 32, 2 << 7)) == 19
    assert fg.check_tuple((256, 256, 32, 64, 128, 4, 16, 1, 512, MFMA32, 32, 16 | 1 << 7)) == 19
    assert fg.check_tuple((128, 64, 16, 64, 64, 2, 4, 4, 128, VALU, 32, 3 << 7)) == 0


def test_residency_request_fields():
    # The config table reports the request through the tuple's opt field;
    # the hinted kernels exist for both variants.
    hinted = [c for c in fg.configs() if c["opt"] & (3 << 7)]
    assert hinted
    for c in hinted:
        assert c["resources_vec"] is not None and c["resources_scalar"] is not None
        b = (c["opt"] >> 7) & 3
        waves = -(-(b + 1) * c["NT"] // 256)
        assert waves <= 8 and (b + 1) * c["lds_bytes"] <= 160 * 1024
    assert fg.check_tuple((96, 64, 24, 32, 64, 2, 16, 1, 192, MFMA32, 0, 0)) == 0


def test_direct_lds_layout_is_conflict_free():
    # The As[m][k] chunk swizzle keeps 128-bit fragment reads free of bank
    # conflicts under both bank models; without it every phase of the read
    # would hit one bank group (8 or 16 rows at the same chunk).
    for t in [(256, 256, 32, 64, 128, 4, 16, 1, 512, MFMA32, 32, 16),
              (128, 128, 16, 32, 64, 2, 16, 1, 512, MFMA32, 32, 16),
              (128, 128, 8, 64, 64, 2, 16, 1, 256, MFMA32, 32, 16)]:
        if fg.check_tuple(t) != 0:
            continue
        for banks in (32, 64):
            r = fg.simulate_tuple(t, banks=banks)
            assert r["status"] == 0, (t, banks, r)
            assert r["dma_read_a_ways"] == 1, (t, banks, r)
            assert r["dma_read_b_ways"] == (1 if banks == 32 else 2)
    # 16x16x4 reads: four 16-lane slots on k-rows 4 apart; the Bs XOR by
    # (k/4 mod 4)*16 built for 64 banks separates all four under both models,
    # the 32-bank one (k/4 mod 2)*16 only the two a 32-bank phase serves.
    for t in [(128, 128, 32, 64, 64, 4, 4, 1, 256, MFMA16, 64, 16),
              (256, 256, 16, 64, 64, 4, 4, 1, 1024, MFMA16, 64, 16),
              (128, 128, 32, 64, 64, 4, 4, 1, 256, MFMA16, 32, 16)]:
        assert fg.check_tuple(t) == 0
        for banks in (32, 64):
            r = fg.simulate_tuple(t, banks=banks)
            assert r["status"] == 0, (t, banks, r)
            assert r["dma_read_a_ways"] == 1, (t, banks, r)
            assert r["dma_read_b_ways"] == (1 if banks == 32 or t[10] == 64 else 2)


@pytest.mark.parametrize("M,N", [(4096, 4096), (4097, 4095), (8192, 2048), (1000, 1500), (256, 256),
                                 (300, 7000), (65, 64), (8192, 8192)])
def test_tile_order_is_a_bijection(M, N):
    for c in fg.configs():
        if c["opt"] & 2 == 0 and (M, N) != (4096, 4096):
            continue
        rows, cols = fg.tile_order(M, N, c["id"])
        tm, tn = -(-M // c["BM"]), -(-N // c["BN"])
        assert len(rows) == tm * tn
        assert sorted(zip(rows, cols)) == [(r, q) for r in range(tm) for q in range(tn)]


def test_xcd_order_gives_each_xcd_a_compact_block():
    c = [x for x in fg.configs() if x["tuple"][:11] == (256, 256, 16, 128, 128, 4, 16, 1, 256, 1, 32)
         and x["opt"] & 2][0]
    rows, cols = fg.tile_order(4096, 4096, c["id"])
    for x in range(8):
        mine = [(rows[i], cols[i]) for i in range(len(rows)) if i % 8 == x]
        # 32 tiles of a 16 x 16 grid in a 4 x 8 block: 4 A row panels, 8 B column panels.
        assert len({r for r, _ in mine}) == 4 and len({q for _, q in mine}) == 8
