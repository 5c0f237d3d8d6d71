"""Sector-charged read accounting.  (Oracle: test infrastructure.)

The pages measure cost as reads: the bytes of each touched 32-byte DRAM
sector, as a percentage of the full model's routed-expert bytes (80 needed
bytes in 4 sectors are charged 128 B) ([zh §前置知识 / 显存带宽受限的解码];
Figure 2).  At the 17.8% budget the reader's reads split into sketch 4.9%,
exact channels 12.3% and recovery map 0.6% ([zh §核心方法]); the sketch takes
about 7% and the recovery map about 0.5% of resident memory
([zh §方法步骤详情]; [ko §어떻게 쓰나]).

Per token and layer the reader touches, in whole 32-B sectors:
  codes   top * nblk * n_screen units (one unit per screened coordinate)
  scales  top * nblk pieces of 2*I fp16 (gate and up scales of one block)
  norms   top pieces of I fp32
  rho     top * nblk pieces of 2*I fp16, only for the expected-error ranking
          of budgets from 28.7% on ([zh §方法步骤详情] decode step (2))
  exact   k channels * 3 rows of H bf16 (gate row, up row, transposed down row)
  b       (top*I - k) skipped channels * rank fp16
  U       H * rank fp16
Dense routed-expert bytes per token: top * 3 * I * H * 2.

Pins (tests/test_oracle_accounting.py): the printed read composition, bytes
per block, resident shares and the full-sketch / partial-screen ratios.
"""
from .sketch import unit_geometry


def _sect(nbytes: int) -> int:
    return -(-nbytes // 32) * 32


def read_bytes(hidden, inter, top, k, rank=32, n_screen=80, block=128, rho=False):
    nblk = hidden // block
    _, unit = unit_geometry(inter)
    r = {
        "codes": top * nblk * n_screen * _sect(unit),
        "scales": top * nblk * _sect(2 * inter * 2),
        "rho": top * nblk * _sect(2 * inter * 2) if rho else 0,
        "norms": top * _sect(inter * 4),
        "exact": k * _sect(3 * hidden * 2),
        "b": (top * inter - k) * _sect(rank * 2),
        "U": _sect(hidden * rank * 2),
    }
    r["sketch"] = r["codes"] + r["scales"] + r["rho"] + r["norms"]
    r["recovery"] = r["b"] + r["U"]
    r["total"] = r["sketch"] + r["exact"] + r["recovery"]
    r["dense"] = top * 3 * inter * hidden * 2
    return r


def resident_bytes(hidden, n_experts, inter, rank=32, block=128):
    nblk = hidden // block
    _, unit = unit_geometry(inter)
    return {
        "experts_bf16": n_experts * 3 * inter * hidden * 2,
        "codes": n_experts * nblk * block * unit,
        "scales": n_experts * nblk * 2 * inter * 2,
        "rho": n_experts * nblk * 2 * inter * 2,
        "norms": n_experts * inter * 4,
        "U": hidden * rank * 2,
        "b": n_experts * inter * rank * 2,
    }
