"""Python face of the plain CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test-suite, the smoke check
and the benchmark's CPU-baseline leg may import this module.  It shares no
code with the GPU library and never imports it.

Arrays are numpy.  Floating inputs are ``float32`` or bf16 bit patterns held
as ``uint16``; results come back as ``float64``.

Sources: "Nectar: Neural Estimation of Cached-Token Attention via Regression"
(Eq. 3.1, Eq. 3.4) and "HashAttention: Semantic Sparsity for Faster Inference"
(Eq. 2; the SCORE / TOPK / GATHER-ATT stages; the fixed windows).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


F32, BF16 = 0, 1


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile an oracle C source with gcc into a shared library (in place)."""
    stale = not os.path.exists(out) or os.path.getmtime(src) > os.path.getmtime(out)
    if force or stale:
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-Wno-unknown-pragmas", src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _dtype_code(*arrays) -> int:
    kinds = {a.dtype for a in arrays}
    if kinds == {np.dtype(np.float32)}:
        return F32
    if kinds == {np.dtype(np.uint16)}:
        return BF16
    raise TypeError("oracle inputs must all be float32 or all uint16 (bf16 bits), got %s" % kinds)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def capacity(n: int, m: int, n_sink: int, n_recent: int) -> int:
    """Most positions the selected set can hold: min(n, m + n_sink + n_recent)."""
    return int(min(n, m + n_sink + n_recent))


class Oracle:
    """The oracle's four calls, bound to one compiled library."""

    def __init__(self, lib_path: str = _LIB_PATH):
        lib = ctypes.CDLL(lib_path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        lib.orc_dense_attn.argtypes = [P, P, P, i32, i32, i32, i32, i32, i64, i64, P, P]
        lib.orc_merge_local.argtypes = [P, i32, P, P, P, P, P, i64, i32, i32, i32, i32, P, P]
        lib.orc_sig_topk.argtypes = [P, P, i32, i32, i32, i64, i64, i64, i64, P, i64, P, P]
        lib.orc_gather_attn.argtypes = [P, P, P, i32, i64, P, P, i64, i32, i32, i32, i32, i64, P, P]
        lib.orc_sig_encode.argtypes = [P, i32, i64, i32, P, i32, P]
        lib.orc_sig_topk_w.argtypes = [P, P, i32, i32, i32, i32, i64, i64, i64, i64, P, i64, P, P]
        for f in (lib.orc_dense_attn, lib.orc_merge_local, lib.orc_sig_topk, lib.orc_gather_attn, lib.orc_sig_encode,
                  lib.orc_sig_topk_w):
            f.restype = ctypes.c_int
        lib.orc_set_threads.argtypes = [i32]
        lib.orc_set_threads.restype = None
        lib.orc_get_threads.argtypes = []
        lib.orc_get_threads.restype = ctypes.c_int
        self.lib = lib
        self.capacity = capacity

    def set_threads(self, n: int) -> None:
        self.lib.orc_set_threads(int(n))

    def get_threads(self) -> int:
        return int(self.lib.orc_get_threads())

    def dense_attn(self, q, k, v):
        """A(q) and alpha(q) of each query against all cached tokens.

        q [B, Hq, d]; k, v [B, Hkv, n, d] (one cache per batch item) or
        [1, Hkv, n, d] / [Hkv, n, d] (one document shared by every batch item).
        Returns (out [B, Hq, d] float64, alpha [B, Hq] float64)."""
        q, k, v = _c(q), _c(k), _c(v)
        if k.ndim == 3:
            k, v = k[None], v[None]
        B, Hq, d = q.shape
        Bk, Hkv, n, dk = k.shape
        assert dk == d and v.shape == k.shape and Bk in (1, B)
        stride = 0 if (Bk == 1 and B != 1) else Hkv * n * d
        out = np.empty((B, Hq, d), np.float64)
        alpha = np.empty((B, Hq), np.float64)
        st = self.lib.orc_dense_attn(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q, k, v), B, Hq, Hkv, d, n,
                                     stride, _ptr(out), _ptr(alpha))
        if st:
            raise ValueError("orc_dense_attn: invalid arguments")
        return out, alpha

    def merge_local(self, q, a_in, alpha_in, k_loc, v_loc, n_loc=None):
        """Exact merge of (A, alpha) with local tokens k_loc, v_loc [B, Hkv, n_loc_max, d].

        n_loc: int array [B] of visible local tokens per batch item (None: all)."""
        q, k_loc, v_loc = _c(q), _c(k_loc), _c(v_loc)
        a_in, alpha_in = _c(a_in, np.float64), _c(alpha_in, np.float64)
        B, Hq, d = q.shape
        _, Hkv, nmax, _ = k_loc.shape
        nl = None if n_loc is None else _c(np.asarray(n_loc), np.int32)
        out = np.empty((B, Hq, d), np.float64)
        alpha = np.empty((B, Hq), np.float64)
        st = self.lib.orc_merge_local(_ptr(q), _dtype_code(q, k_loc, v_loc), _ptr(a_in), _ptr(alpha_in),
                                      _ptr(k_loc), _ptr(v_loc), _ptr(nl), nmax, B, Hq, Hkv, d,
                                      _ptr(out), _ptr(alpha))
        if st:
            raise ValueError("orc_merge_local: invalid arguments")
        return out, alpha

    def sig_score_topk(self, key_sigs, q_sigs, m, n_sink, n_recent, cap=None, want_scores=False):
        """SCORE + TOPK.  key_sigs [B, Hkv, n] uint32, q_sigs [B, Hq] uint32.

        Returns (idx [B, Hq, cap] int32 ascending, -1 padded; count [B, Hq] int32;
        scores [B, Hq, n] int8 or None)."""
        ks = _c(np.asarray(key_sigs).view(np.uint32) if np.asarray(key_sigs).dtype == np.int32 else key_sigs,
                np.uint32)
        qs = _c(np.asarray(q_sigs).view(np.uint32) if np.asarray(q_sigs).dtype == np.int32 else q_sigs,
                np.uint32)
        B, Hkv, n = ks.shape
        Hq = qs.shape[1]
        if cap is None:
            cap = capacity(n, m, n_sink, n_recent)
        idx = np.empty((B, Hq, cap), np.int32)
        count = np.empty((B, Hq), np.int32)
        scores = np.empty((B, Hq, n), np.int8) if want_scores else None
        st = self.lib.orc_sig_topk(_ptr(ks), _ptr(qs), B, Hq, Hkv, n, int(m), int(n_sink), int(n_recent),
                                   _ptr(idx), int(cap), _ptr(count), _ptr(scores))
        if st:
            raise ValueError("orc_sig_topk: invalid arguments or cap too small")
        return idx, count, scores

    def gather_attn(self, q, k, v, idx, count):
        """Attention of each query head over its selected positions only.

        q [B, Hq, d]; k, v [B, Hkv, n, d] (or shared [1, Hkv, n, d]);
        idx [B, Hq, cap] int32; count [B, Hq] int32."""
        q, k, v = _c(q), _c(k), _c(v)
        if k.ndim == 3:
            k, v = k[None], v[None]
        idx, count = _c(idx, np.int32), _c(count, np.int32)
        B, Hq, d = q.shape
        Bk, Hkv, n, _ = k.shape
        stride = 0 if (Bk == 1 and B != 1) else Hkv * n * d
        cap = idx.shape[2]
        out = np.empty((B, Hq, d), np.float64)
        alpha = np.empty((B, Hq), np.float64)
        st = self.lib.orc_gather_attn(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q, k, v), stride, _ptr(idx),
                                      _ptr(count), cap, B, Hq, Hkv, d, n, _ptr(out), _ptr(alpha))
        if st:
            raise ValueError("orc_gather_attn: invalid arguments")
        return out, alpha

    def sig_score_topk_w(self, key_sigs, q_sigs, m, n_sink, n_recent, cap=None, want_scores=False):
        """SCORE + TOPK over codes of W words.  key_sigs [B, Hkv, n, W] uint32, q_sigs [B, Hq, W] uint32.

        Returns (idx [B, Hq, cap] int32, count [B, Hq] int32, scores [B, Hq, n] int16 or None)."""
        ks = _c(np.asarray(key_sigs).view(np.uint32), np.uint32)
        qs = _c(np.asarray(q_sigs).view(np.uint32), np.uint32)
        B, Hkv, n, W = ks.shape
        Hq = qs.shape[1]
        assert qs.shape == (B, Hq, W)
        if cap is None:
            cap = capacity(n, m, n_sink, n_recent)
        idx = np.empty((B, Hq, cap), np.int32)
        count = np.empty((B, Hq), np.int32)
        scores = np.empty((B, Hq, n), np.int16) if want_scores else None
        st = self.lib.orc_sig_topk_w(_ptr(ks), _ptr(qs), W, B, Hq, Hkv, n, int(m), int(n_sink), int(n_recent),
                                     _ptr(idx), int(cap), _ptr(count), _ptr(scores))
        if st:
            raise ValueError("orc_sig_topk_w: invalid arguments or cap too small")
        return idx, count, scores

    def sig_encode(self, x, R):
        """Random-projection codes of the rows of x [..., d] (bf16 bit patterns or float32):
        bit b = (x . R[:, b] > 0), as an fma chain in double.  R: [d, bits] float32, bits <= 32.
        Returns uint32 [...]."""
        x = _c(x)
        R = _c(np.asarray(R, np.float32), np.float32)
        d, bits = R.shape
        assert x.shape[-1] == d
        lead = x.shape[:-1]
        rows = int(np.prod(lead)) if lead else 1
        codes = np.empty(rows, np.uint32)
        st = self.lib.orc_sig_encode(_ptr(x), _dtype_code(x), rows, d, _ptr(R), bits, _ptr(codes))
        if st:
            raise ValueError("orc_sig_encode: invalid arguments")
        return codes.reshape(lead)


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c (compiled on first use if needed)."""
    global _default
    if _default is None:
        build()
        _default = Oracle(_LIB_PATH)
    return _default


def dense_attn(*a, **kw):
    return default().dense_attn(*a, **kw)


def merge_local(*a, **kw):
    return default().merge_local(*a, **kw)


def sig_score_topk(*a, **kw):
    return default().sig_score_topk(*a, **kw)


def sig_encode(*a, **kw):
    return default().sig_encode(*a, **kw)


def gather_attn(*a, **kw):
    return default().gather_attn(*a, **kw)


def set_threads(n: int) -> None:
    default().set_threads(n)


def get_threads() -> int:
    return default().get_threads()
