"""Pins for the sector-charged read accounting against the pages' printed numbers."""
import json
import os

import pytest

from oracle.accounting import read_bytes, resident_bytes
from oracle.sketch import unit_geometry

H, E, I, TOP = 2048, 128, 768, 8


@pytest.fixture(scope="module")
def printed(golden_dir):
    return json.load(open(os.path.join(golden_dir, "printed_numbers.json")))


def _pct(v, d):
    return 100.0 * v / d


def test_read_composition_at_17_8(printed):
    p = printed["read_composition_17_8"]
    r = read_bytes(H, I, TOP, p["k"])
    d = r["dense"]
    assert round(_pct(r["sketch"], d), 1) == p["sketch_pct"]
    assert round(_pct(r["exact"], d), 1) == p["exact_pct"]
    assert round(_pct(r["recovery"], d), 1) == p["recovery_pct"]
    assert round(_pct(r["total"], d), 1) == p["total_pct"]
    lo, hi = printed["recovery_reads_pp"]["lo"], printed["recovery_reads_pp"]["hi"]
    assert lo <= _pct(r["recovery"], d) <= hi
    assert r["total"] == 13_460_224 and d == 75_497_472


def test_budget_12_8(printed):
    p = printed["budget_12_8"]
    r = read_bytes(H, I, TOP, p["k"])
    assert round(_pct(r["total"], r["dense"]), 1) == p["total_pct"]


def test_candidates(printed):
    assert TOP * I == printed["candidates"]["value"]


def test_bytes_per_block(printed):
    p = printed["bytes_per_block"]
    assert 128 * 2 == p["bf16_bytes"]
    _, unit = unit_geometry(I)
    per_row_block = 128 * unit / (2 * I) + 2 + 2  # codes share + fp16 scale + fp16 rho
    assert abs(per_row_block - p["approx_sketch_bytes"]) <= p["tol"]


def test_resident_shares(printed):
    r = resident_bytes(H, E, I)
    ex = r["experts_bf16"]
    assert round(_pct(r["codes"] + r["scales"], ex)) == printed["resident_sketch_pct"]["approx"]
    assert round(_pct(r["U"] + r["b"], ex), 1) == printed["resident_recovery_pct"]["approx"]


def test_full_sketch_share_and_partial_screen_gain(printed):
    fs, ps = printed["full_sketch_share_pct"], printed["partial_screen_more_exact_pct"]
    shares = []
    for k in (756, 445):
        budget = read_bytes(H, I, TOP, k)["total"]
        kf = max(kk for kk in range(TOP * I + 1)
                 if read_bytes(H, I, TOP, kk, n_screen=128)["total"] <= budget)
        full = read_bytes(H, I, TOP, kf, n_screen=128)
        shares.append(_pct(full["sketch"], full["total"]))
        if k == ps["at_budget_k"]:
            gain = 100.0 * (k / kf - 1.0)
            assert ps["lo"] <= gain <= ps["hi"]
    assert abs(min(shares) - fs["lo"]) <= fs["tol_pp"]
    assert abs(max(shares) - fs["hi"]) <= fs["tol_pp"]
