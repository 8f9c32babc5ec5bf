"""Host-side arithmetic of bench.py: the algorithmic work per stage and the
whole-path floor, checked against figures worked out by hand for the 64K text
shape (batch 1, 8 heads, L 65536, d 128, 1024 buckets, chunks of 64, 4 rounds,
bf16) and the float32 tiny shape.  No GPU is touched."""
import math

import bench
from efficient_long_sequence_lsh_amd import workloads as W

N_TEXT = 1 * 8 * 65536


def test_stage_work_text_64k():
    w = W.WORKLOADS["text_64k"]
    work = bench.stage_work(w)
    # 2 d flops per projection, b/2 projections per round, 4 rounds
    assert work["hash"]["flops"] == N_TEXT * 4 * (2 * 128 * 512)
    # rounds 0..2: qk and v rows (2 x 256 B) + perm entry, then a compact row of
    # 128 12-bit values (192 B; its z and scale exponent in the values' own bits)
    assert work["attend"]["bytes"] == N_TEXT * 3 * ((256 + 256 + 4) + 192)
    # last round: its own gather, the three earlier rows, the bf16 output row
    assert work["combine"]["bytes"] == N_TEXT * ((256 + 256 + 4) + 3 * 192 + 256)
    # d = 64 keeps float16 rows (a 96-byte row would still touch two 64-byte sectors)
    img = W.WORKLOADS["image_12k"]
    n_img = 8 * 8 * 12288
    assert bench.stage_work(img)["attend"]["bytes"] == n_img * 7 * ((128 + 128 + 4) + 128)
    assert bench.sort_path(w) == "tiles"
    assert work["sort"]["bytes"] == N_TEXT * 4 * 12


def test_path_roofline_text_64k():
    w = W.WORKLOADS["text_64k"]
    p = bench.path_roofline(0.8, w)
    hash_ms = N_TEXT * 4 * 128 * 1024 / 2.5e15 * 1e3           # 0.10995 ms
    hbm_ms = (N_TEXT * 3 * 708 + N_TEXT * 1348 + N_TEXT * 48) / 8e12 * 1e3
    assert math.isclose(p["stage_floor_ms"]["hash"], round(hash_ms, 4), abs_tol=1e-4)
    assert math.isclose(p["t_roof_ms"], hash_ms + hbm_ms, abs_tol=2e-4)
    assert math.isclose(p["frac"], (hash_ms + hbm_ms) / 0.8, abs_tol=2e-4)
    assert 0.34 < p["t_roof_ms"] < 0.35


def test_float32_hash_priced_at_the_vector_peak():
    w = W.WORKLOADS["tiny_1k"]
    flops = bench.stage_work(w)["hash"]["flops"]
    p = bench.path_roofline(1.0, w)
    assert math.isclose(p["stage_floor_ms"]["hash"], round(flops / 157.3e12 * 1e3, 4), abs_tol=1e-4)
    rf = bench.roofline_for("hash", 1.0, w)
    assert rf["bound"] == "alu" and rf["peak"] == 157.3
    assert "executed_mfma_frac" not in rf


def test_backward_work_text_64k():
    w = W.WORKLOADS["text_64k"]
    flops, nbytes = bench.backward_work(w)
    assert flops == N_TEXT * 4 * 7 * 2 * 128 * 128
    # stats 524 B; per round 768 B of rows + 12 B of perm, Z, D; float32 gradient rows:
    # 1 KB written in round 0, 1 KB read and 1 KB written in rounds 1..3
    assert nbytes == N_TEXT * (524 + 4 * 780 + 1024 + 3 * 2048)


def test_other_resource_text_64k():
    """The hash against HBM and chunk attention against the bf16 matrix peak:
    the hash reads each 256-byte qk row once and writes 4 ids of 4 bytes; a
    chunk of 64 queries against its 128-key window does 2 x 64 x 128 x 128
    flops for S and as many for O, i.e. 4 x 128 x 128 per query and round."""
    w = W.WORKLOADS["text_64k"]
    h = bench.other_resource("hash", 1.0, w)["hbm"]
    assert math.isclose(h["achieved"], round(N_TEXT * (256 + 16) / 1e-3 / 1e9, 1))
    assert h["peak"] == 8000.0
    a = bench.other_resource("attend", 1.0, w)["mfma"]
    assert math.isclose(a["achieved"], round(N_TEXT * 3 * 4 * 128 * 128 / 1e-3 / 1e12, 2))
    c = bench.other_resource("combine", 1.0, w)["mfma"]
    assert math.isclose(c["achieved"], round(N_TEXT * 4 * 128 * 128 / 1e-3 / 1e12, 2))
    assert a["peak"] == c["peak"] == 2500.0
    assert bench.other_resource("sort", 1.0, w) == {}
    # float32 inputs: attention runs on float32 matrix cores
    assert bench.other_resource("attend", 1.0, W.WORKLOADS["tiny_1k"])["mfma"]["peak"] == 157.3
