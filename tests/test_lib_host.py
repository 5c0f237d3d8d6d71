"""CPU-side tests of libcfr.so: symbols, validation, accounting, and the
host pack checked bit for bit against the oracle.  No GPU is used."""
import ctypes
import os
import re

import numpy as np
import pytest

from calibration_free_channel_amd import Config, pack_host, read_bytes, sizes
from calibration_free_channel_amd._lib import SIGNATURES, CfrConfig, CfrError, load
from oracle import OracleReader, read_bytes as oracle_read_bytes
from oracle.sketch import unit_geometry
from synth import make_layer, workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    txt = open(os.path.join(ROOT, "include", "cfr.h")).read()
    return sorted(set(re.findall(r"^(?:int|void|const char\*)\s+(cfr_[a-z0-9_]+)\s*\(", txt, re.M)))


def test_library_exports_every_declared_symbol():
    lib = load()
    declared = _declared_symbols()
    assert declared, "no declarations found"
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(SIGNATURES), "binding and header disagree"


def _cfg(**kw):
    base = dict(hidden=256, n_experts=16, inter=64, top=2)
    base.update(kw)
    return Config(**base)


def test_sizes_match_the_layout():
    for inter in (64, 768, 1536, 7):
        s = sizes(_cfg(inter=inter, hidden=2048, n_experts=8))
        lp, unit = unit_geometry(inter)
        assert (s["half_bytes"], s["unit_bytes"]) == (lp, unit)
        assert s["codes_bytes"] == 8 * 16 * 128 * unit
        assert s["n_cand"] == 2 * inter


@pytest.mark.parametrize("k", [0, 445, 756, 6144])
def test_read_bytes_match_oracle_accounting(k):
    cfg = Config(hidden=2048, n_experts=128, inter=768, top=8)
    got = read_bytes(cfg, k)
    ref = oracle_read_bytes(2048, 768, 8, k)
    for key in ("codes", "scales", "norms", "exact", "b", "total", "dense"):
        assert got[key] == ref[key], key
    assert got["u"] == ref["U"]


@pytest.mark.parametrize("k", [0, 1234, 6144])
def test_read_bytes_with_rho_match_oracle_accounting(k):
    # the expected-error ranking reads the whole sketch and rho_b as well
    cfg = Config(hidden=2048, n_experts=128, inter=768, top=8, n_screen=128, ranking=1)
    got = read_bytes(cfg, k)
    ref = oracle_read_bytes(2048, 768, 8, k, n_screen=128, rho=True)
    for key in ("codes", "scales", "rho", "norms", "exact", "b", "total", "dense"):
        assert got[key] == ref[key], key
    assert read_bytes(Config(hidden=2048, n_experts=128, inter=768, top=8), k)["rho"] == 0


@pytest.mark.parametrize("bad", [dict(hidden=200), dict(hidden=0), dict(top=0), dict(top=17),
                                 dict(n_screen=0), dict(n_screen=129), dict(rank=65), dict(rank=12),
                                 dict(max_batch=0), dict(inter=0), dict(inter=5000),
                                 dict(n_experts=1, top=2), dict(ranking=2), dict(ranking=-1),
                                 dict(ranking=1, n_screen=80)])
def test_invalid_configs_rejected(bad):
    with pytest.raises(CfrError) as ei:
        sizes(_cfg(**bad))
    assert ei.value.code in (-1, -4)


def test_invalid_k_rejected():
    with pytest.raises(CfrError):
        read_bytes(_cfg(), -1)
    with pytest.raises(CfrError):
        read_bytes(_cfg(), 129)


def test_null_pointers_rejected():
    lib = load()
    cfg = _cfg().c()
    assert lib.cfr_pack_host(ctypes.byref(cfg), None, None, None, None, None, None, None) == -1
    assert lib.cfr_build_reader(None, None, None, None, None, ctypes.byref(ctypes.c_void_p())) == -1
    assert b"NULL" in lib.cfr_last_error()
    assert lib.cfr_reader_decode(None, None, None, None, 1, 0, None, None) == -1
    lib.cfr_reader_free(None)  # NULL-safe


def _compare_pack(wl, n_experts=None, seed_layer=0):
    s = wl.shape
    layer = make_layer(wl, seed_layer)
    E = n_experts or s.n_experts
    g, u, d = layer["gate"][:E], layer["up"][:E], layer["down"][:E]
    cfg = Config(hidden=s.hidden, n_experts=E, inter=s.inter, top=min(s.top, E),
                 rot_seed=wl.rot_seed)
    got = pack_host(cfg, g, u, d)
    ref = OracleReader(s.hidden, E, s.inter, min(s.top, E), g, u, d, rank=4, rot_seed=wl.rot_seed)
    assert np.array_equal(got["codes"], ref.units)
    assert np.array_equal(got["scales"], ref.alpha_bits)
    assert np.array_equal(got["rho"], ref.rho_bits)
    assert np.array_equal(got["norms"], ref.norms)


def test_host_pack_rejects_nonfinite_weights():
    # a NaN or an infinity in any weight is rejected before any work
    from synth import make_layer, workload
    wl = workload("tiny")
    s = wl.shape
    L = make_layer(wl)
    cfg = Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top)
    for name, bits in (("gate", 0x7FC0), ("up", 0x7F80), ("down", 0xFF80)):
        bad = {k: v.copy() for k, v in L.items()}
        bad[name].reshape(-1)[17] = bits
        with pytest.raises(CfrError) as ei:
            pack_host(cfg, bad["gate"], bad["up"], bad["down"])
        assert ei.value.code == -1


def test_host_pack_bit_exact_tiny():
    _compare_pack(workload("tiny"))


def test_host_pack_bit_exact_qwen3_30b_shape_subset():
    # the Qwen3-30B-A3B layer shape (hidden 2048, intermediate 768) on 3 experts
    _compare_pack(workload("qwen3-30b-a3b"), n_experts=3)


@pytest.mark.slow
def test_host_pack_bit_exact_qwen3_235b_shape_subset():
    _compare_pack(workload("qwen3-235b-a22b"), n_experts=2)


def test_exact_bits_rules_and_4bit_accounting():
    from calibration_free_channel_amd import Config, RANK_EXPECTED_ERROR, read_bytes
    from calibration_free_channel_amd._lib import CfrError
    base = dict(hidden=2048, n_experts=128, inter=768, top=8)
    with pytest.raises(CfrError):
        read_bytes(Config(**base, exact_bits=8), 10)
    with pytest.raises(CfrError):
        read_bytes(Config(**base, exact_bits=4, n_screen=128, ranking=RANK_EXPECTED_ERROR), 10)
    b16 = read_bytes(Config(**base), 756)
    b4 = read_bytes(Config(**base, exact_bits=4), 756)
    # a 4-bit row of 2048 weights: 1024 code bytes, 16 fp16 scales, 16 zero
    # points (1072 bytes); a kept channel's three rows, 3216 bytes, touch 101
    # 32-byte sectors
    assert b4["exact"] == 756 * 3232
    assert b4["dense"] == 8 * 3 * 768 * 1072
    for f in ("codes", "scales", "norms", "b", "u"):
        assert b4[f] == b16[f]
    assert read_bytes(Config(**base, exact_bits=0), 756) == b16
