"""Python binding of liblcda (ctypes): every C-ABI call of include/lcda.h under the same name.

Only argument marshalling happens here: every tensor is checked (device,
contiguity, dtype, shape; ValueError before any launch), outputs and the
workspace are allocated with torch on the tensors' device unless given, and the
call is enqueued on torch's current HIP stream.  Every step of the path runs in
the HIP kernels of liblcda.so; there is no fallback of any kind: if the library
is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblcda.so")

LCDA_F32, LCDA_BF16 = 0, 1
STATUS = {0: "LCDA_OK", 1: "LCDA_EINVAL", 2: "LCDA_EUNSUPPORTED", 3: "LCDA_EWORKSPACE", 4: "LCDA_EHIP"}

# Every symbol include/lcda.h declares.
EXPORTS = ("cached_attn_lse", "lse_merge_local", "sig_score_topk", "gather_attn",
           "lcda_ws_bytes_cached_attn_lse", "lcda_ws_bytes_lse_merge_local",
           "lcda_ws_bytes_sig_score_topk", "lcda_ws_bytes_gather_attn",
           "lcda_last_error", "lcda_version", "lcda_set_tuning", "lcda_get_tuning",
           "dense_decode_step", "lcda_ws_bytes_dense_decode_step", "sig_encode", "sig_score_topk_q",
           "sig_score_topk_w", "lcda_ws_bytes_sig_score_topk_w", "dense_decode_step_noalloc",
           "lcda_noalloc_scratch_bytes", "sparse_decode_step", "lcda_ws_bytes_sparse_decode_step",
           "lcda_stream_read")

_lib = None


class LcdaError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__("%s failed: %s: %s" % (fn, STATUS.get(status, status), text))
        self.status = status


def load(path: str = LIB_PATH):
    """Open liblcda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("liblcda.so is not built (%s); run __graft_entry__.build() or "
                           "python -m long_context_decode_attn_amd.build" % path)
    lib = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.cached_attn_lse.argtypes = [P, P, P, i32, i32, i32, i32, i64, i64, i32, P, P, P, sz, P]
    lib.lse_merge_local.argtypes = [P, P, P, P, P, P, i64, i32, i32, i32, i32, i32, P, P, P, sz, P]
    lib.sig_score_topk.argtypes = [P, P, i32, i32, i32, i64, i64, i64, i64, P, i64, P, P, P, sz, P]
    lib.sig_score_topk_q.argtypes = [P, P, i32, P, i32, i32, i32, i32, i64, i64, i64, i64, P, i64, P, P, P, P, sz, P]
    lib.sig_encode.argtypes = [P, i32, i64, i64, i64, P, i32, P, i64, P]
    lib.sig_score_topk_w.argtypes = [P, P, i32, i32, i32, i32, i64, i64, i64, i64, P, i64, P, P, P, sz, P]
    lib.lcda_ws_bytes_sig_score_topk_w.argtypes = [i32, i32, i64]
    lib.lcda_ws_bytes_sig_score_topk_w.restype = sz
    lib.gather_attn.argtypes = [P, P, P, i64, P, P, i64, i32, i32, i32, i32, i64, i32, P, P, P, sz, P]
    for f in (lib.cached_attn_lse, lib.lse_merge_local, lib.sig_score_topk, lib.gather_attn):
        f.restype = ctypes.c_int
    lib.lcda_ws_bytes_cached_attn_lse.argtypes = [i32, i32, i32, i32, i64, i64]
    lib.lcda_ws_bytes_lse_merge_local.argtypes = [i32, i32, i32, i32, i64]
    lib.lcda_ws_bytes_sig_score_topk.argtypes = [i32, i32, i32, i64]
    lib.lcda_ws_bytes_gather_attn.argtypes = [i32, i32, i32, i32, i64]
    for f in (lib.lcda_ws_bytes_cached_attn_lse, lib.lcda_ws_bytes_lse_merge_local,
              lib.lcda_ws_bytes_sig_score_topk, lib.lcda_ws_bytes_gather_attn):
        f.restype = ctypes.c_size_t
    lib.lcda_last_error.restype = ctypes.c_char_p
    lib.lcda_last_error.argtypes = []
    lib.lcda_version.restype = ctypes.c_char_p
    lib.lcda_version.argtypes = []
    lib.dense_decode_step.argtypes = [P, P, P, i64, i64, P, P, P, i64, i32, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    lib.dense_decode_step.restype = ctypes.c_int
    lib.lcda_ws_bytes_dense_decode_step.argtypes = [i32, i32, i32, i32, i64, i64, i64]
    lib.lcda_ws_bytes_dense_decode_step.restype = ctypes.c_size_t
    lib.dense_decode_step_noalloc.argtypes = [P, P, P, i64, i64, P, P, P, i64, i32, i32, i32, i32, i32, P, P, P]
    lib.dense_decode_step_noalloc.restype = ctypes.c_int
    lib.lcda_noalloc_scratch_bytes.argtypes = []
    lib.lcda_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.sparse_decode_step.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i32, i64, i32, i64, i64, i64, P, i64, P, P,
                                       P, P, sz, P]
    lib.sparse_decode_step.restype = ctypes.c_int
    lib.lcda_ws_bytes_sparse_decode_step.argtypes = [i32, i32, i32, i32, i64, i64]
    lib.lcda_ws_bytes_sparse_decode_step.restype = ctypes.c_size_t
    lib.lcda_stream_read.argtypes = [P, sz, i32, P, ctypes.c_uint32, P]
    lib.lcda_stream_read.restype = ctypes.c_int
    lib.lcda_set_tuning.argtypes = [ctypes.c_char_p, i64]
    lib.lcda_set_tuning.restype = ctypes.c_int
    lib.lcda_get_tuning.argtypes = [ctypes.c_char_p]
    lib.lcda_get_tuning.restype = i64
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise LcdaError(fn, status, load().lcda_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LCDA_F32
    if t.dtype == torch.bfloat16:
        return LCDA_BF16
    raise TypeError("q/K/V must be float32 or bfloat16, got %s" % t.dtype)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


# Every tensor that reaches a kernel is checked here first (device, contiguity,
# dtype, shape): a host tensor or a short buffer must never become a device
# pointer.  Failures raise ValueError before any launch.
_CODES = (torch.int32, torch.uint32)


def _tensor(t, name: str, dev, dtypes=None, shape=None):
    _need(isinstance(t, torch.Tensor), "%s must be a tensor" % name)
    _need(t.device == dev, "%s must be on %s, got %s" % (name, dev, t.device))
    _need(t.is_contiguous(), "%s must be contiguous" % name)
    if dtypes is not None:
        _need(t.dtype in dtypes, "%s must be %s, got %s" % (name, " or ".join(str(d) for d in dtypes), t.dtype))
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), "%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t


def _out(t, name: str, shape, dev, dtype=torch.float32):
    """A caller-provided output (checked) or a new one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    return _tensor(t, name, dev, (dtype,), shape)


def _gpu(t, name: str):
    _need(isinstance(t, torch.Tensor), "%s must be a tensor" % name)
    _need(t.is_cuda, "%s must be on a GPU, got %s" % (name, t.device))
    return t.device


def _ws(nbytes: int, device, ws):
    if ws is not None:
        _tensor(ws, "ws", device)
        _need(ws.numel() * ws.element_size() >= nbytes, "workspace too small: need %d bytes" % nbytes)
        return ws
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _as_kv(k: torch.Tensor, B: int, dev=None, name="K/V"):
    """K/V as [Bkv, Hkv, n, d]; returns (tensor4d, kv_batch_stride in elements)."""
    _need(isinstance(k, torch.Tensor), "%s must be a tensor" % name)
    if k.dim() == 3:
        k = k.unsqueeze(0)
    _need(k.dim() == 4, "%s must be [B, Hkv, n, d] or [Hkv, n, d]" % name)
    if dev is not None:
        _tensor(k, name, dev)
    _need(k.is_contiguous(), "%s must be contiguous" % name)
    Bk = k.shape[0]
    _need(Bk in (1, B), "%s batch %d must be 1 (shared document) or B = %d" % (name, Bk, B))
    stride = 0 if (Bk == 1 and B != 1) else k.shape[1] * k.shape[2] * k.shape[3]
    return k, stride


def _query(q, name="q"):
    """q [B, Hq, d] on a GPU, float32 or bfloat16, contiguous; returns (device, B, Hq, d)."""
    dev = _gpu(q, name)
    _need(q.dim() == 3, "%s must be [B, Hq, d]" % name)
    _tensor(q, name, dev, (torch.float32, torch.bfloat16))
    return (dev,) + tuple(q.shape)


def _kv_pair(k, v, B, dev, dtype):
    k, stride = _as_kv(k, B, dev, "K")
    v, _ = _as_kv(v, B, dev, "V")
    _need(v.shape == k.shape, "K and V shapes differ")
    _need(k.dtype == dtype and v.dtype == dtype, "q, K, V must share a dtype")
    return k, v, stride


def _locals(k_loc, v_loc, n_loc, B, dev, dtype):
    _tensor(k_loc, "k_loc", dev, (dtype,))
    _tensor(v_loc, "v_loc", dev, (dtype,))
    _need(k_loc.dim() == 4 and k_loc.shape[0] == B and k_loc.shape == v_loc.shape, "k_loc/v_loc must be [B, Hkv, n, d]")
    if n_loc is not None:
        _tensor(n_loc, "n_loc", dev, (torch.int32,))
        _need(n_loc.numel() == B, "n_loc must be int32 [B] on the GPU")


def ws_bytes_cached_attn_lse(B, Hq, Hkv, d, n, kv_batch_stride) -> int:
    return int(load().lcda_ws_bytes_cached_attn_lse(B, Hq, Hkv, d, n, kv_batch_stride))


def ws_bytes_lse_merge_local(B, Hq, Hkv, d, n_loc_max) -> int:
    return int(load().lcda_ws_bytes_lse_merge_local(B, Hq, Hkv, d, n_loc_max))


def ws_bytes_sig_score_topk(B, Hq, Hkv, n) -> int:
    return int(load().lcda_ws_bytes_sig_score_topk(B, Hq, Hkv, n))


def ws_bytes_gather_attn(B, Hq, Hkv, d, cap) -> int:
    return int(load().lcda_ws_bytes_gather_attn(B, Hq, Hkv, d, cap))


def cached_attn_lse(q, k, v, out=None, alpha=None, ws=None):
    """A(q) [B, Hq, d] fp32 and alpha(q) [B, Hq] fp32 of q [B, Hq, d] against K, V.

    K, V: [B, Hkv, n, d] (one cache per batch item) or [1, Hkv, n, d] (one
    document shared by all B items)."""
    lib = load()
    dev, B, Hq, d = _query(q)
    k, v, stride = _kv_pair(k, v, B, dev, q.dtype)
    Hkv, n = k.shape[1], k.shape[2]
    out = _out(out, "out", (B, Hq, d), dev)
    alpha = _out(alpha, "alpha", (B, Hq), dev)
    nb = lib.lcda_ws_bytes_cached_attn_lse(B, Hq, Hkv, d, n, stride)
    w = _ws(nb, q.device, ws)
    st = lib.cached_attn_lse(_p(q), _p(k), _p(v), B, Hq, Hkv, d, n, stride, _dtype_code(q),
                             _p(out), _p(alpha), _p(w), w.numel() * w.element_size(), _stream(q.device))
    _check("cached_attn_lse", st)
    return out, alpha


def lse_merge_local(q, a_in, alpha_in, k_loc, v_loc, n_loc=None, out=None, alpha_out=None, ws=None,
                    want_alpha=True):
    """Exact merge of (A, alpha) with local tokens k_loc, v_loc [B, Hkv, n_loc_max, d].

    n_loc: int32 tensor [B] on the GPU (None: all n_loc_max tokens visible)."""
    lib = load()
    dev, B, Hq, d = _query(q)
    _tensor(a_in, "a_in", dev, (torch.float32,), (B, Hq, d))
    _tensor(alpha_in, "alpha_in", dev, (torch.float32,), (B, Hq))
    _locals(k_loc, v_loc, n_loc, B, dev, q.dtype)
    Hkv, nmax = k_loc.shape[1], k_loc.shape[2]
    out = _out(out, "out", (B, Hq, d), dev)
    if want_alpha or alpha_out is not None:
        alpha_out = _out(alpha_out, "alpha_out", (B, Hq), dev)
    nb = lib.lcda_ws_bytes_lse_merge_local(B, Hq, Hkv, d, nmax)
    w = _ws(nb, q.device, ws)
    st = lib.lse_merge_local(_p(q), _p(a_in), _p(alpha_in), _p(k_loc), _p(v_loc), _p(n_loc), nmax, B, Hq, Hkv, d,
                             _dtype_code(q), _p(out), _p(alpha_out), _p(w), w.numel() * w.element_size(),
                             _stream(q.device))
    _check("lse_merge_local", st)
    return out, alpha_out


def ws_bytes_dense_decode_step(B, Hq, Hkv, d, n, kv_batch_stride, n_loc_max) -> int:
    return int(load().lcda_ws_bytes_dense_decode_step(B, Hq, Hkv, d, n, kv_batch_stride, n_loc_max))


def dense_decode_step(q, k, v, k_loc, v_loc, n_loc=None, out=None, alpha_out=None, a_doc=None, alpha_doc=None,
                      ws=None, want_alpha=True):
    """cached_attn_lse followed by lse_merge_local, fused into one pass where possible.

    Returns (out, alpha_out); a_doc / alpha_doc (both or neither) receive the cached-only (A, alpha)."""
    lib = load()
    dev, B, Hq, d = _query(q)
    k, v, stride = _kv_pair(k, v, B, dev, q.dtype)
    _locals(k_loc, v_loc, n_loc, B, dev, q.dtype)
    Hkv, n = k.shape[1], k.shape[2]
    nmax = k_loc.shape[2]
    out = _out(out, "out", (B, Hq, d), dev)
    if want_alpha or alpha_out is not None:
        alpha_out = _out(alpha_out, "alpha_out", (B, Hq), dev)
    _need((a_doc is None) == (alpha_doc is None), "a_doc and alpha_doc go together")
    if a_doc is not None:
        _tensor(a_doc, "a_doc", dev, (torch.float32,), (B, Hq, d))
        _tensor(alpha_doc, "alpha_doc", dev, (torch.float32,), (B, Hq))
    nb = lib.lcda_ws_bytes_dense_decode_step(B, Hq, Hkv, d, n, stride, nmax)
    w = _ws(nb, q.device, ws)
    st = lib.dense_decode_step(_p(q), _p(k), _p(v), stride, n, _p(k_loc), _p(v_loc), _p(n_loc), nmax, B, Hq, Hkv, d,
                               _dtype_code(q), _p(out), _p(alpha_out), _p(a_doc), _p(alpha_doc), _p(w),
                               w.numel() * w.element_size(), _stream(q.device))
    _check("dense_decode_step", st)
    return out, alpha_out


def dense_decode_step_noalloc(q, k, v, k_loc, v_loc, n_loc=None, out=None, alpha_out=None, want_alpha=True):
    """dense_decode_step with the library's static scratch array instead of a workspace (the call itself
    allocates nothing; outputs are allocated here unless given).  Returns (out, alpha_out)."""
    lib = load()
    dev, B, Hq, d = _query(q)
    k, v, stride = _kv_pair(k, v, B, dev, q.dtype)
    _locals(k_loc, v_loc, n_loc, B, dev, q.dtype)
    Hkv, n = k.shape[1], k.shape[2]
    nmax = k_loc.shape[2]
    out = _out(out, "out", (B, Hq, d), dev)
    if want_alpha or alpha_out is not None:
        alpha_out = _out(alpha_out, "alpha_out", (B, Hq), dev)
    st = lib.dense_decode_step_noalloc(_p(q), _p(k), _p(v), stride, n, _p(k_loc), _p(v_loc), _p(n_loc), nmax, B, Hq,
                                       Hkv, d, _dtype_code(q), _p(out), _p(alpha_out), _stream(q.device))
    _check("dense_decode_step_noalloc", st)
    return out, alpha_out


def noalloc_scratch_bytes() -> int:
    return int(load().lcda_noalloc_scratch_bytes())


def capacity(n: int, m: int, n_sink: int, n_recent: int) -> int:
    return int(min(n, m + n_sink + n_recent))


def sig_score_topk(key_sigs, q_sigs, m, n_sink, n_recent, cap=None, want_scores=False, idx=None, count=None,
                   ws=None):
    """SCORE + TOPK.  key_sigs [B, Hkv, n], q_sigs [B, Hq] (int32 storage of uint32 codes).

    Returns (idx [B, Hq, cap] int32, count [B, Hq] int32, scores [B, Hq, n] int8 or None)."""
    lib = load()
    dev = _gpu(key_sigs, "key_sigs")
    _need(key_sigs.dim() == 3, "key_sigs must be [B, Hkv, n]")
    _tensor(key_sigs, "key_sigs", dev, _CODES)
    B, Hkv, n = key_sigs.shape
    _need(isinstance(q_sigs, torch.Tensor) and q_sigs.dim() == 2 and q_sigs.shape[0] == B, "q_sigs must be [B, Hq]")
    _tensor(q_sigs, "q_sigs", dev, (key_sigs.dtype,))
    Hq = q_sigs.shape[1]
    cap = capacity(n, m, n_sink, n_recent) if cap is None else int(cap)
    idx = _out(idx, "idx", (B, Hq, cap), dev, torch.int32)
    count = _out(count, "count", (B, Hq), dev, torch.int32)
    scores = torch.empty((B, Hq, n), dtype=torch.int8, device=dev) if want_scores else None
    nb = lib.lcda_ws_bytes_sig_score_topk(B, Hq, Hkv, n)
    w = _ws(nb, dev, ws)
    st = lib.sig_score_topk(_p(key_sigs), _p(q_sigs), B, Hq, Hkv, n, int(m), int(n_sink), int(n_recent), _p(idx),
                            cap, _p(count), _p(scores), _p(w), w.numel() * w.element_size(), _stream(dev))
    _check("sig_score_topk", st)
    return idx, count, scores


def sig_score_topk_q(key_sigs, q, R, m, n_sink, n_recent, cap=None, want_scores=False, idx=None, count=None,
                     q_sigs=None, ws=None):
    """SCORE + TOPK with the query codes encoded at the head of the scan from q [B, Hq, 128] and R [128, bits]
    (fp32).  Returns (idx, count, scores or None, q_sigs [B, Hq] int32 storage of uint32 codes)."""
    lib = load()
    dev = _gpu(key_sigs, "key_sigs")
    _need(key_sigs.dim() == 3, "key_sigs must be [B, Hkv, n]")
    _tensor(key_sigs, "key_sigs", dev, _CODES)
    B, Hkv, n = key_sigs.shape
    _need(isinstance(q, torch.Tensor) and q.dim() == 3 and q.shape[0] == B and q.shape[2] == 128,
          "q must be [B, Hq, 128]")
    _tensor(q, "q", dev, (torch.float32, torch.bfloat16))
    _need(isinstance(R, torch.Tensor) and R.dim() == 2 and R.shape[0] == 128, "R: [128, bits] fp32")
    _tensor(R, "R", dev, (torch.float32,))
    Hq = q.shape[1]
    cap = capacity(n, m, n_sink, n_recent) if cap is None else int(cap)
    idx = _out(idx, "idx", (B, Hq, cap), dev, torch.int32)
    count = _out(count, "count", (B, Hq), dev, torch.int32)
    q_sigs = _out(q_sigs, "q_sigs", (B, Hq), dev, torch.int32)
    scores = torch.empty((B, Hq, n), dtype=torch.int8, device=dev) if want_scores else None
    nb = lib.lcda_ws_bytes_sig_score_topk(B, Hq, Hkv, n)
    w = _ws(nb, dev, ws)
    st = lib.sig_score_topk_q(_p(key_sigs), _p(q), _dtype_code(q), _p(R), R.shape[1], B, Hq, Hkv, n, int(m),
                              int(n_sink), int(n_recent), _p(idx), cap, _p(count), _p(scores), _p(q_sigs), _p(w),
                              w.numel() * w.element_size(), _stream(dev))
    _check("sig_score_topk_q", st)
    return idx, count, scores, q_sigs


def sig_score_topk_w(key_sigs, q_sigs, m, n_sink, n_recent, cap=None, want_scores=False, idx=None, count=None,
                     ws=None):
    """SCORE + TOPK over codes of W words.  key_sigs [B, Hkv, n, W], q_sigs [B, Hq, W] (int32 storage).

    Returns (idx [B, Hq, cap] int32, count [B, Hq] int32, scores [B, Hq, n] int16 or None)."""
    lib = load()
    dev = _gpu(key_sigs, "key_sigs")
    _need(key_sigs.dim() == 4, "key_sigs must be [B, Hkv, n, W]")
    _tensor(key_sigs, "key_sigs", dev, _CODES)
    B, Hkv, n, W = key_sigs.shape
    _need(isinstance(q_sigs, torch.Tensor) and q_sigs.dim() == 3, "q_sigs must be [B, Hq, W]")
    Hq = q_sigs.shape[1]
    _tensor(q_sigs, "q_sigs", dev, (key_sigs.dtype,), (B, Hq, W))
    cap = capacity(n, m, n_sink, n_recent) if cap is None else int(cap)
    idx = _out(idx, "idx", (B, Hq, cap), dev, torch.int32)
    count = _out(count, "count", (B, Hq), dev, torch.int32)
    scores = torch.empty((B, Hq, n), dtype=torch.int16, device=dev) if want_scores else None
    nb = lib.lcda_ws_bytes_sig_score_topk_w(B, Hq, n)
    w = _ws(nb, dev, ws)
    st = lib.sig_score_topk_w(_p(key_sigs), _p(q_sigs), W, B, Hq, Hkv, n, int(m), int(n_sink), int(n_recent), _p(idx),
                              cap, _p(count), _p(scores), _p(w), w.numel() * w.element_size(), _stream(dev))
    _check("sig_score_topk_w", st)
    return idx, count, scores


def sig_encode(x, R, codes=None):
    """Random-projection codes (T_map) of rows of 128 values, R [128, bits] fp32.

    x contiguous [..., 128] gives codes [...] (int32 storage of uint32), new unless given.  x may also be a
    [B, H, r, 128] view into a cache (rows contiguous, heads evenly strided, e.g. K[:, :, n_old:n_old + r]); codes
    must then be the matching [B, H, r] view into the key codes (e.g. key_sigs[:, :, n_old:n_old + r])."""
    lib = load()
    dev = _gpu(x, "x")
    _need(x.dtype in (torch.float32, torch.bfloat16), "x must be float32 or bfloat16")
    _need(isinstance(R, torch.Tensor) and R.dim() == 2 and R.shape[0] == 128, "R: [128, bits] fp32")
    _tensor(R, "R", dev, (torch.float32,))
    _need(x.shape[-1] == 128 and x.stride(-1) == 1, "rows of x must hold 128 contiguous values")
    if codes is not None:
        _need(isinstance(codes, torch.Tensor) and codes.device == dev and codes.dtype in _CODES,
              "codes must be 32-bit on %s" % dev)
    if x.is_contiguous():
        lead = x.shape[:-1]
        rows = x.numel() // 128
        codes = torch.empty(lead, dtype=torch.int32, device=dev) if codes is None else codes
        _need(codes.is_contiguous() and codes.numel() == rows, "codes must be contiguous, one per row")
        g, rpg, xs, cs = 1, rows, 0, 0
    else:
        _need(x.dim() == 4 and x.stride(2) == 128 and x.stride(0) == x.shape[1] * x.stride(1),
              "a strided x must be [B, H, r, 128] with contiguous rows and evenly strided heads")
        _need(codes is not None and tuple(codes.shape) == tuple(x.shape[:3]) and codes.stride(2) == 1
              and codes.stride(0) == codes.shape[1] * codes.stride(1), "codes must be the matching [B, H, r] view")
        g, rpg, xs, cs = x.shape[0] * x.shape[1], x.shape[2], x.stride(1), codes.stride(1)
    st = lib.sig_encode(_p(x), _dtype_code(x), g, rpg, xs, _p(R), R.shape[1], _p(codes), cs, _stream(x.device))
    _check("sig_encode", st)
    return codes


def gather_attn(q, k, v, idx, count, out=None, alpha=None, ws=None, want_alpha=True):
    """Attention of each query head over its selected positions idx[:, :, :count] only."""
    lib = load()
    dev, B, Hq, d = _query(q)
    k, v, stride = _kv_pair(k, v, B, dev, q.dtype)
    _need(isinstance(idx, torch.Tensor) and idx.dim() == 3 and tuple(idx.shape[:2]) == (B, Hq),
          "idx must be [B, Hq, cap]")
    _tensor(idx, "idx", dev, (torch.int32,))
    _tensor(count, "count", dev, (torch.int32,), (B, Hq))
    Hkv, n = k.shape[1], k.shape[2]
    cap = idx.shape[2]
    out = _out(out, "out", (B, Hq, d), dev)
    if want_alpha or alpha is not None:
        alpha = _out(alpha, "alpha", (B, Hq), dev)
    nb = lib.lcda_ws_bytes_gather_attn(B, Hq, Hkv, d, cap)
    w = _ws(nb, q.device, ws)
    st = lib.gather_attn(_p(q), _p(k), _p(v), stride, _p(idx), _p(count), cap, B, Hq, Hkv, d, n, _dtype_code(q),
                         _p(out), _p(alpha), _p(w), w.numel() * w.element_size(), _stream(q.device))
    _check("gather_attn", st)
    return out, alpha


def ws_bytes_sparse_decode_step(B, Hq, Hkv, d, n, cap) -> int:
    return int(load().lcda_ws_bytes_sparse_decode_step(B, Hq, Hkv, d, n, cap))


def sparse_decode_step(key_sigs, q_sigs, q, k, v, m, n_sink, n_recent, cap=None, idx=None, count=None, out=None,
                       alpha=None, ws=None, want_alpha=True):
    """SCORE + TOPK + GATHER-ATT in one launch where possible.  key_sigs [B, Hkv, n], q_sigs [B, Hq] (int32
    storage of uint32 codes); q [B, Hq, 128]; K, V [B, Hkv, n, 128] (or a shared [1, Hkv, n, 128]).

    Returns (idx [B, Hq, cap] int32, count [B, Hq] int32, out [B, Hq, 128] fp32, alpha [B, Hq] fp32)."""
    lib = load()
    dev, B, Hq, d = _query(q)
    k, v, stride = _kv_pair(k, v, B, dev, q.dtype)
    Hkv, n = k.shape[1], k.shape[2]
    _tensor(key_sigs, "key_sigs", dev, _CODES, (B, Hkv, n))
    _tensor(q_sigs, "q_sigs", dev, (key_sigs.dtype,), (B, Hq))
    cap = capacity(n, m, n_sink, n_recent) if cap is None else int(cap)
    idx = _out(idx, "idx", (B, Hq, cap), dev, torch.int32)
    count = _out(count, "count", (B, Hq), dev, torch.int32)
    out = _out(out, "out", (B, Hq, d), dev)
    if want_alpha or alpha is not None:
        alpha = _out(alpha, "alpha", (B, Hq), dev)
    nb = lib.lcda_ws_bytes_sparse_decode_step(B, Hq, Hkv, d, n, cap)
    w = _ws(nb, dev, ws)
    st = lib.sparse_decode_step(_p(key_sigs), _p(q_sigs), _p(q), _p(k), _p(v), stride, B, Hq, Hkv, d, n, _dtype_code(q),
                                int(m), int(n_sink), int(n_recent), _p(idx), cap, _p(count), _p(out), _p(alpha), _p(w),
                                w.numel() * w.element_size(), _stream(dev))
    _check("sparse_decode_step", st)
    return idx, count, out, alpha


def stream_read(buf: torch.Tensor, workgroups: int, sink: torch.Tensor = None) -> None:
    """The streaming-read probe (lcda_stream_read) over all of buf (a contiguous GPU tensor whose size in bytes is
    a multiple of 16): enqueued on torch's current stream; time it with events."""
    dev = _gpu(buf, "buf")
    _tensor(buf, "buf", dev)
    nbytes = buf.numel() * buf.element_size()
    _need(nbytes % 16 == 0, "buf must hold a multiple of 16 bytes")
    sink = _out(sink, "sink", (1,), dev, torch.int32)
    _check("lcda_stream_read", load().lcda_stream_read(_p(buf), nbytes, int(workgroups), _p(sink), 0x9E3779B9,
                                                       _stream(dev)))


def set_tuning(key: str, value: int) -> None:
    """Launch-shape knob (see lcda_set_tuning in include/lcda.h)."""
    _check("lcda_set_tuning", load().lcda_set_tuning(key.encode(), int(value)))


def get_tuning(key: str) -> int:
    return int(load().lcda_get_tuning(key.encode()))


def version() -> str:
    return load().lcda_version().decode()
