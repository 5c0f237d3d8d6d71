"""Python binding of the reader: argument marshalling around libcfr.so.

Every step of the decode path runs in the library's HIP kernels; this module
only checks shapes and dtypes, takes device pointers from torch tensors and
passes the current HIP stream.  There is no fallback: without the built
library every call raises.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from . import _lib
from ._lib import CfrConfig, CfrReadStats, CfrSizes, check, load

DEFAULT_ROT_SEED = 0x5EED_0000_CAFE_F00D
RANK_SCORE = 0            # output-unit score, partial screen (low budgets)
RANK_EXPECTED_ERROR = 1   # whole sketch, expected squared error with rho (from 28.7%)


@dataclass(frozen=True)
class Config:
    hidden: int
    n_experts: int
    inter: int
    top: int
    rank: int = 32
    n_screen: int = 80
    max_batch: int = 1
    device: int = 0
    rot_seed: int = DEFAULT_ROT_SEED
    ranking: int = RANK_SCORE
    exact_bits: int = 16  # 16: native BF16 exact rows; 4: a 4-bit checkpoint (Reader.build_q4)

    def c(self) -> CfrConfig:
        return CfrConfig(self.hidden, self.n_experts, self.inter, self.top, self.rank,
                         self.n_screen, self.max_batch, self.device, self.rot_seed & (2 ** 64 - 1),
                         self.ranking, self.exact_bits)


def sizes(cfg: Config) -> dict:
    s = CfrSizes()
    check(load().cfr_sizes_of(ctypes.byref(cfg.c()), ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in CfrSizes._fields_}


def read_bytes(cfg: Config, k: int) -> dict:
    s = CfrReadStats()
    check(load().cfr_read_bytes(ctypes.byref(cfg.c()), int(k), ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in CfrReadStats._fields_}


def read_bytes_batch(cfg: Config, expert_ids, sel, kept, k: int) -> dict:
    """Distinct 32-byte sectors one batched decode call reads (the library's
    union count), from the call's expert ids [B][top], screened coordinates
    [B][nblk][n_screen] and kept candidates [B][k] (host arrays, as
    decode_debug returns them)."""
    ids = np.ascontiguousarray(expert_ids, dtype=np.int32)
    sel = np.ascontiguousarray(sel, dtype=np.uint8)
    kept = np.ascontiguousarray(np.asarray(kept)[:, :k], dtype=np.int32)
    B = ids.shape[0]
    if ids.shape != (B, cfg.top) or sel.shape != (B, cfg.hidden // 128, cfg.n_screen) or kept.shape != (B, k):
        raise ValueError("expert_ids [B][top], sel [B][nblk][n_screen] and kept [B][k] expected")
    s = CfrReadStats()
    check(load().cfr_read_bytes_batch(ctypes.byref(cfg.c()), B, int(k), _ptr(ids), _ptr(sel),
                                      _ptr(kept) if k > 0 else None, ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in CfrReadStats._fields_}


def read_bytes_shared(cfg: Config, expert_ids, sel, n_kept: int) -> dict:
    """Distinct 32-byte sectors one batch-shared decode call reads, from the
    call's expert ids [B][top], screened coordinates [B][nblk][n_screen]
    (host arrays) and the number of kept union candidates."""
    ids = np.ascontiguousarray(expert_ids, dtype=np.int32)
    sel = np.ascontiguousarray(sel, dtype=np.uint8)
    B = ids.shape[0]
    if ids.shape != (B, cfg.top) or sel.shape != (B, cfg.hidden // 128, cfg.n_screen):
        raise ValueError("expert_ids [B][top] and sel [B][nblk][n_screen] expected")
    s = CfrReadStats()
    check(load().cfr_read_bytes_shared(ctypes.byref(cfg.c()), B, _ptr(ids), _ptr(sel), int(n_kept),
                                       ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in CfrReadStats._fields_}


def _u16(a, shape, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16 or a.shape != tuple(shape):
        raise ValueError(f"{name}: expected uint16 (bf16 bits) of shape {tuple(shape)}, "
                         f"got {a.dtype} {a.shape}")
    return a


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def pack_host(cfg: Config, gate, up, down) -> dict:
    """Host-only sketch pack and down norms (load steps 1 and 2), no device used."""
    E, I, H = cfg.n_experts, cfg.inter, cfg.hidden
    gate = _u16(gate, (E, I, H), "gate")
    up = _u16(up, (E, I, H), "up")
    down = _u16(down, (E, H, I), "down")
    sz = sizes(cfg)
    nblk = sz["n_blocks"]
    codes = np.empty((E, nblk, 128, sz["unit_bytes"]), dtype=np.uint8)
    scales = np.empty((E, nblk, 2, I), dtype=np.uint16)
    rho = np.empty((E, nblk, 2, I), dtype=np.uint16)
    norms = np.empty((E, I), dtype=np.float32)
    check(load().cfr_pack_host(ctypes.byref(cfg.c()), _ptr(gate), _ptr(up), _ptr(down),
                               _ptr(codes), _ptr(scales), _ptr(rho), _ptr(norms)))
    return {"codes": codes, "scales": scales, "rho": rho, "norms": norms}


def _torch():
    import torch
    return torch


def _dev_tensor(t, dtype, shape, name, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if t.device.index != device:
        raise ValueError(f"{name}: on device {t.device}, reader is on device {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


class Reader:
    """One built layer.  Owns device memory until close()."""

    def __init__(self, handle: ctypes.c_void_p, cfg: Config):
        self._h = handle
        self.cfg = cfg
        self._sizes = sizes(cfg)

    # -- construction ------------------------------------------------------
    @classmethod
    def build(cls, cfg: Config, gate, up, down, router=None) -> "Reader":
        """Load-time work (rotation, ternary pack, norms, SVD, transpose) for one layer."""
        E, I, H = cfg.n_experts, cfg.inter, cfg.hidden
        gate = _u16(gate, (E, I, H), "gate")
        up = _u16(up, (E, I, H), "up")
        down = _u16(down, (E, H, I), "down")
        if router is not None:
            router = _u16(router, (E, H), "router")
        h = ctypes.c_void_p()
        check(load().cfr_build_reader(ctypes.byref(cfg.c()), _ptr(gate), _ptr(up), _ptr(down),
                                      _ptr(router), ctypes.byref(h)))
        return cls(h, cfg)

    @classmethod
    def build_q4(cls, cfg: Config, rows, router=None) -> "Reader":
        """A reader over a 4-bit checkpoint: rows uint8 [E][I][3][R], each
        channel's gate row, up row and down column as 4-bit row records of
        R = roundup(H/2 + 3 H/128, 16) bytes (codes, fp16 group scales, zero
        points; cfr_build_reader_q4).  cfg.exact_bits must be 4."""
        E, I, H = cfg.n_experts, cfg.inter, cfg.hidden
        R = -(-(H // 2 + 3 * (H // 128)) // 16) * 16
        rows = np.ascontiguousarray(rows)
        if rows.dtype != np.uint8 or rows.shape != (E, I, 3, R):
            raise ValueError(f"rows: expected uint8 of shape {(E, I, 3, R)}, got {rows.dtype} {rows.shape}")
        if router is not None:
            router = _u16(router, (E, H), "router")
        h = ctypes.c_void_p()
        check(load().cfr_build_reader_q4(ctypes.byref(cfg.c()), _ptr(rows), _ptr(router), ctypes.byref(h)))
        return cls(h, cfg)

    def clone(self) -> "Reader":
        h = ctypes.c_void_p()
        check(load().cfr_reader_clone(self._h, ctypes.byref(h)))
        return Reader(h, self.cfg)

    def close(self):
        if self._h is not None and self._h.value:
            load().cfr_reader_free(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- decode --------------------------------------------------------------
    def _stream(self, stream):
        torch = _torch()
        s = stream if stream is not None else torch.cuda.current_stream(self.cfg.device)
        return ctypes.c_void_p(s.cuda_stream)

    def _args(self, x, ids, w):
        torch = _torch()
        if x.dim() != 2:
            raise ValueError("x must be [batch, hidden]")
        B = x.shape[0]
        c = self.cfg
        return (B, _dev_tensor(x, torch.float32, (B, c.hidden), "x", c.device),
                _dev_tensor(ids, torch.int32, (B, c.top), "expert_ids", c.device),
                _dev_tensor(w, torch.float32, (B, c.top), "gate_w", c.device))

    def decode(self, x, expert_ids, gate_w, k: int, out=None, stream=None, residual=None):
        """The reader's output for x [batch, hidden]; with `residual` (a
        [batch, hidden] float32 tensor, which may be `out` but not x) the
        output plus residual, added in the last kernel."""
        torch = _torch()
        B, px, pi, pw = self._args(x, expert_ids, gate_w)
        if out is None:
            out = torch.empty((B, self.cfg.hidden), dtype=torch.float32, device=x.device)
        py = _dev_tensor(out, torch.float32, (B, self.cfg.hidden), "out", self.cfg.device)
        if residual is None:
            check(load().cfr_reader_decode(self._h, px, pi, pw, B, int(k), py, self._stream(stream)))
        else:
            pr = _dev_tensor(residual, torch.float32, (B, self.cfg.hidden), "residual", self.cfg.device)
            check(load().cfr_reader_decode_residual(self._h, px, pi, pw, B, int(k), pr, py,
                                                    self._stream(stream)))
        return out

    def decode_noalloc(self, x, expert_ids, gate_w, k: int, out, stream=None):
        """cfr_reader_decode_noalloc: the decode with its per-call buffers in
        the library's static device array (no allocation in the call); `out`
        [batch, hidden] float32 is required.  Calls overlapping on one device
        race (they share the array)."""
        torch = _torch()
        B, px, pi, pw = self._args(x, expert_ids, gate_w)
        py = _dev_tensor(out, torch.float32, (B, self.cfg.hidden), "out", self.cfg.device)
        check(load().cfr_reader_decode_noalloc(self._h, px, pi, pw, B, int(k), py, self._stream(stream)))
        return out

    def decode_shared(self, x, expert_ids, gate_w, k: int, out=None, stream=None, debug=False):
        """cfr_reader_decode_shared: one top-k of k channels for the whole
        batch over its distinct routed experts (at most 8 tokens).  Returns y
        [batch, hidden]; with debug=True a dict with y, the batch scores
        "bscore" [u * inter], the kept union candidates "kept" and the union's
        experts "experts" (ascending), u = their number."""
        torch = _torch()
        B, px, pi, pw = self._args(x, expert_ids, gate_w)
        c, dev = self.cfg, x.device
        if out is None:
            out = torch.empty((B, c.hidden), dtype=torch.float32, device=dev)
        py = _dev_tensor(out, torch.float32, (B, c.hidden), "out", c.device)
        if not debug:
            check(load().cfr_reader_decode_shared(self._h, px, pi, pw, B, int(k), py, None, None, None,
                                                  self._stream(stream)))
            return out
        bs = torch.empty((B * c.top * c.inter,), dtype=torch.float32, device=dev)
        kp = torch.empty((max(int(k), 1),), dtype=torch.int32, device=dev)
        ex = torch.empty((1 + B * c.top,), dtype=torch.int32, device=dev)
        check(load().cfr_reader_decode_shared(self._h, px, pi, pw, B, int(k), py,
                                              ctypes.c_void_p(bs.data_ptr()), ctypes.c_void_p(kp.data_ptr()),
                                              ctypes.c_void_p(ex.data_ptr()), self._stream(stream)))
        torch.cuda.synchronize(dev)
        u = int(ex[0].item())
        return {"y": out, "bscore": bs[:u * c.inter], "kept": kp[:min(int(k), u * c.inter)],
                "experts": ex[1:1 + u]}

    def decode_debug(self, x, expert_ids, gate_w, k: int, stream=None) -> dict:
        torch = _torch()
        B, px, pi, pw = self._args(x, expert_ids, gate_w)
        c, dev = self.cfg, x.device
        nc = c.top * c.inter
        o = {
            "y": torch.empty((B, c.hidden), dtype=torch.float32, device=dev),
            "xrot": torch.empty((B, c.hidden), dtype=torch.float32, device=dev),
            "sel": torch.empty((B, c.hidden // 128, c.n_screen), dtype=torch.uint8, device=dev),
            "ghat": torch.empty((B, nc), dtype=torch.float32, device=dev),
            "vhat": torch.empty((B, nc), dtype=torch.float32, device=dev),
            "score": torch.empty((B, nc), dtype=torch.float32, device=dev),
            "kept": torch.empty((B, max(int(k), 1)), dtype=torch.int32, device=dev),
        }
        p = {n: ctypes.c_void_p(t.data_ptr()) for n, t in o.items()}
        check(load().cfr_reader_decode_debug(self._h, px, pi, pw, B, int(k), p["y"], p["xrot"],
                                             p["sel"], p["ghat"], p["vhat"], p["score"],
                                             p["kept"], self._stream(stream)))
        o["kept"] = o["kept"][:, :int(k)]
        return o

    STAGES = ("screen", "select", "reduce")

    def decode_profile(self, x, expert_ids, gate_w, k: int, out=None, stream=None) -> dict:
        """Decode with an event after every stage; returns {stage: microseconds}.

        Synchronises the host; for measurement only."""
        torch = _torch()
        B, px, pi, pw = self._args(x, expert_ids, gate_w)
        if out is None:
            out = torch.empty((B, self.cfg.hidden), dtype=torch.float32, device=x.device)
        py = _dev_tensor(out, torch.float32, (B, self.cfg.hidden), "out", self.cfg.device)
        us = (ctypes.c_float * len(self.STAGES))()
        check(load().cfr_reader_decode_profile(self._h, px, pi, pw, B, int(k), py, us,
                                               self._stream(stream)))
        return dict(zip(self.STAGES, list(us)))

    def decode_stage(self, stage: int, x, expert_ids, gate_w, k: int, out=None, stream=None):
        """Launch one decode stage's kernel alone (0 screen, 1 select, 2 reduce);
        for timing a kernel in isolation.  y is the decode's only when the three
        stages run in order for the same inputs."""
        torch = _torch()
        B, px, pi, pw = self._args(x, expert_ids, gate_w)
        if out is None:
            out = torch.empty((B, self.cfg.hidden), dtype=torch.float32, device=x.device)
        py = _dev_tensor(out, torch.float32, (B, self.cfg.hidden), "out", self.cfg.device)
        check(load().cfr_reader_decode_stage(self._h, int(stage), px, pi, pw, B, int(k), py,
                                             self._stream(stream)))
        return out

    def route(self, x, ids_out=None, w_out=None, stream=None, norm_out=None, norm_eps=1e-6):
        """Softmax top-k routing of x [batch, hidden] with the router weights
        given at build time: (expert_ids int32 [batch, top], gate_w float32
        [batch, top]), by weight descending.  With norm_out (a [batch, hidden]
        float32 tensor) the router reads RMSNorm(x) (unit weights, norm_eps)
        and writes it to norm_out."""
        torch = _torch()
        if x.dim() != 2:
            raise ValueError("x must be [batch, hidden]")
        B, c = x.shape[0], self.cfg
        px = _dev_tensor(x, torch.float32, (B, c.hidden), "x", c.device)
        if ids_out is None:
            ids_out = torch.empty((B, c.top), dtype=torch.int32, device=x.device)
        if w_out is None:
            w_out = torch.empty((B, c.top), dtype=torch.float32, device=x.device)
        pi = _dev_tensor(ids_out, torch.int32, (B, c.top), "ids_out", c.device)
        pw = _dev_tensor(w_out, torch.float32, (B, c.top), "w_out", c.device)
        pn = None if norm_out is None else _dev_tensor(norm_out, torch.float32, (B, c.hidden), "norm_out",
                                                          c.device)
        check(load().cfr_reader_route(self._h, px, B, float(norm_eps), pn, pi, pw, self._stream(stream)))
        return ids_out, w_out

    def dense(self, x, expert_ids, gate_w, out=None, stream=None, residual=None):
        torch = _torch()
        B, px, pi, pw = self._args(x, expert_ids, gate_w)
        if out is None:
            out = torch.empty((B, self.cfg.hidden), dtype=torch.float32, device=x.device)
        py = _dev_tensor(out, torch.float32, (B, self.cfg.hidden), "out", self.cfg.device)
        if residual is None:
            check(load().cfr_dense_decode(self._h, px, pi, pw, B, py, self._stream(stream)))
        else:
            pr = _dev_tensor(residual, torch.float32, (B, self.cfg.hidden), "residual", self.cfg.device)
            check(load().cfr_dense_decode_residual(self._h, px, pi, pw, B, pr, py, self._stream(stream)))
        return out

    # -- state ----------------------------------------------------------------
    def export(self) -> dict:
        c, sz = self.cfg, self._sizes
        E, I, H, nblk = c.n_experts, c.inter, c.hidden, sz["n_blocks"]
        o = {
            "codes": np.empty((E, nblk, 128, sz["unit_bytes"]), dtype=np.uint8),
            "scales": np.empty((E, nblk, 2, I), dtype=np.uint16),
            "rho": np.empty((E, nblk, 2, I), dtype=np.uint16),
            "norms": np.empty((E, I), dtype=np.float32),
            "U": np.empty((H, c.rank), dtype=np.uint16),
            "b": np.empty((E, I, c.rank), dtype=np.uint16),
            "sigma": np.empty((H,), dtype=np.float32),
        }
        check(load().cfr_reader_export(self._h, *(_ptr(o[n]) for n in
                                                  ("codes", "scales", "rho", "norms", "U", "b",
                                                   "sigma"))))
        return o

    def status(self) -> int:
        f = ctypes.c_int32()
        check(load().cfr_reader_status(self._h, ctypes.byref(f)))
        return f.value
