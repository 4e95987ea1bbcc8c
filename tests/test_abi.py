"""The C-ABI library: it loads, exports every symbol include/lcda.h declares, and rejects
invalid arguments before any HIP call (so these run without a GPU: no compute call is made)."""
import ctypes
import os
import re

import pytest

from long_context_decode_attn_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    text = open(os.path.join(ROOT, "include", "lcda.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        pytest.skip("liblcda.so not built")
    return ops.load()


def test_every_declared_symbol_is_exported(lib):
    syms = header_symbols()
    assert set(syms) == set(ops.EXPORTS), syms
    for s in syms:
        assert hasattr(lib, s), s
    assert lib.lcda_version().decode().count(".") == 2


P = ctypes.c_void_p


def fake(addr=0x10000):
    return ctypes.c_void_p(addr)   # aligned non-null pointer that is never dereferenced


def call_dense(lib, **kw):
    a = dict(q=fake(), k=fake(), v=fake(), B=1, Hq=4, Hkv=1, d=128, n=64, stride=0, dtype=1,
             out=fake(), alpha=fake(), ws=fake(), ws_bytes=1 << 30)
    a.update(kw)
    return lib.cached_attn_lse(a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["d"], a["n"], a["stride"],
                               a["dtype"], a["out"], a["alpha"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code,text", [
    (dict(d=64), 2, "d = 64"),
    (dict(Hq=6, Hkv=4), 1, "multiple"),
    (dict(Hkv=0), 1, "positive"),
    (dict(B=-1), 1, "B = -1"),
    (dict(n=-1), 1, "n = -1"),
    (dict(n=1 << 31), 2, "INT32_MAX"),
    (dict(dtype=7), 2, "dtype"),
    (dict(q=None), 1, "q is NULL"),
    (dict(out=ctypes.c_void_p(0x10004)), 1, "aligned"),
    (dict(stride=100), 1, "kv_batch_stride"),
    (dict(ws_bytes=16), 3, "workspace"),
    (dict(ws=None), 3, "workspace"),
])
def test_cached_attn_lse_rejects(lib, kw, code, text):
    assert call_dense(lib, **kw) == code
    assert text in lib.lcda_last_error().decode()


def test_merge_and_topk_and_gather_reject(lib):
    # lse_merge_local: out aliasing a_in
    st = lib.lse_merge_local(fake(), fake(0x20000), fake(), fake(), fake(), None, 8, 1, 4, 1, 128, 1,
                             fake(0x20000), None, fake(), 1 << 30, None)
    assert st == 1 and "alias" in lib.lcda_last_error().decode()
    # sig_score_topk: cap too small, negative m, too many heads per group
    st = lib.sig_score_topk(fake(), fake(), 1, 4, 1, 1000, 10, 2, 2, fake(), 13, fake(), None, fake(), 1 << 30, None)
    assert st == 1 and "cap" in lib.lcda_last_error().decode()
    st = lib.sig_score_topk(fake(), fake(), 1, 4, 1, 1000, -1, 2, 2, fake(), 13, fake(), None, fake(), 1 << 30, None)
    assert st == 1
    st = lib.sig_score_topk(fake(), fake(), 1, 16, 1, 1000, 10, 2, 2, fake(), 14, fake(), None, fake(), 1 << 30, None)
    assert st == 2
    st = lib.sig_score_topk(fake(), fake(), 1, 4, 1, 1000, 10, 2, 2, fake(), 14, fake(), None, fake(), 8, None)
    assert st == 3
    # gather_attn: null idx
    st = lib.gather_attn(fake(), fake(), fake(), 0, None, fake(), 16, 1, 4, 1, 128, 100, 1, fake(), None, fake(),
                         1 << 30, None)
    assert st == 1 and "idx" in lib.lcda_last_error().decode()


def test_workspace_sizes(lib):
    assert lib.lcda_ws_bytes_cached_attn_lse(1, 32, 8, 128, 61440, 8 * 61440 * 128) > 0
    assert lib.lcda_ws_bytes_cached_attn_lse(1, 32, 8, 64, 61440, 0) == 0
    # One 33-bin histogram per query head and chunk (and two for the window
    # parts); by default about topk_wgs workgroups of whole 4096-position
    # sub-chunks: 512 / (8 x 8) = 8 chunks here.
    assert lib.lcda_get_tuning(b"topk_subs") == 0 and lib.lcda_get_tuning(b"topk_wgs") == 512
    chunks = 8
    assert lib.lcda_ws_bytes_sig_score_topk(8, 32, 8, 131072) >= 8 * 32 * chunks * 33 * 4
    assert lib.lcda_ws_bytes_gather_attn(8, 32, 8, 128, 4352) > 0
    assert lib.lcda_ws_bytes_lse_merge_local(1, 32, 8, 128, 256) > 0


def test_empty_batch_is_a_no_op(lib):
    assert call_dense(lib, B=0, q=None, out=None, alpha=None, ws=None, ws_bytes=0) == 0


def test_sig_encode_rejects(lib):
    """T_map: bad bit counts, dtypes, strides and alignments are refused before any HIP call."""
    R = fake()
    def call(**kw):
        a = dict(x=fake(), dtype=1, groups=2, rpg=4, xs=4 * 128, R=R, bits=32, codes=fake(), cs=4)
        a.update(kw)
        return lib.sig_encode(a["x"], a["dtype"], a["groups"], a["rpg"], a["xs"], a["R"], a["bits"], a["codes"],
                              a["cs"], None)
    assert call(bits=0) == 1 and b"bits" in lib.lcda_last_error()
    assert call(bits=33) == 1
    assert call(dtype=5) == 2
    assert call(xs=3 * 128) == 1 and b"overlap" in lib.lcda_last_error()
    assert call(cs=3) == 1
    assert call(xs=4 * 128 + 4) == 1 and b"multiple of 8" in lib.lcda_last_error()
    assert call(codes=ctypes.c_void_p(0x10002)) == 1 and b"4-byte" in lib.lcda_last_error()
    assert call(x=None) == 1
    assert call(groups=1 << 20, rpg=1 << 12, xs=(1 << 12) * 128, cs=1 << 12) == 2   # 2^32 rows
    assert b"INT32_MAX" in lib.lcda_last_error()
    assert call(groups=0, x=None, R=None, codes=None) == 0   # nothing to do


def test_sig_score_topk_q_rejects(lib):
    st = lib.sig_score_topk_q(fake(), fake(), 1, fake(), 40, 1, 4, 1, 1000, 10, 2, 2, fake(), 14, fake(), None,
                              fake(), fake(), 1 << 30, None)
    assert st == 1 and b"bits" in lib.lcda_last_error()
    st = lib.sig_score_topk_q(fake(), None, 1, fake(), 32, 1, 4, 1, 1000, 10, 2, 2, fake(), 14, fake(), None,
                              fake(), fake(), 1 << 30, None)
    assert st == 1 and b"q is NULL" in lib.lcda_last_error()


def test_dense_decode_step_noalloc_rejects(lib):
    """The no-allocation step refuses shapes whose workspace exceeds its static array, and bad arguments,
    before any HIP call (the array's address is looked up only for a call that will run)."""
    cap = lib.lcda_noalloc_scratch_bytes()
    assert 0 < cap < (16 << 20)
    B, Hq, Hkv, n = 128, 32, 8, 61440   # a shared document read by 128 items: 21 MB of partial states
    assert lib.lcda_ws_bytes_dense_decode_step(B, Hq, Hkv, 128, n, 0, 512) > cap
    st = lib.dense_decode_step_noalloc(fake(), None, None, 0, n, None, None, None, 512, B, Hq, Hkv, 128,
                                       1, fake(), None, None)
    assert st == 2 and b"scratch" in lib.lcda_last_error()
    st = lib.dense_decode_step_noalloc(fake(), fake(), fake(), 0, 1000, fake(), fake(), None, 64, 9000, 1, 1, 128,
                                       1, fake(), None, None)
    assert st == 2 and b"8192" in lib.lcda_last_error()
    # a shape that fits, with a NULL input: the argument check, not the array, answers
    st = lib.dense_decode_step_noalloc(fake(), None, fake(), 0, 1000, fake(), fake(), None, 64, 2, 8, 2, 128, 1,
                                       fake(), None, None)
    assert st == 1 and b"k is NULL" in lib.lcda_last_error()
    assert lib.dense_decode_step_noalloc(None, None, None, 0, 1000, None, None, None, 64, 0, 8, 2, 128, 1, None, None,
                                         None) == 0


def test_workspace_sizes_of_an_empty_batch(lib):
    """B = 0 (no rows) sizes to a small workspace for every kernel choice, a shared document included."""
    for stride in (0, 2 * 1000 * 128):
        assert lib.lcda_ws_bytes_cached_attn_lse(0, 8, 2, 128, 1000, stride) >= 0
        assert lib.lcda_ws_bytes_dense_decode_step(0, 8, 2, 128, 1000, stride, 64) >= 0


@pytest.mark.parametrize("which", ["m", "n_sink", "n_recent"])
def test_topk_rejects_huge_counts_before_summing(lib, which):
    """m, n_sink and n_recent beyond INT32_MAX are refused before they are added up (a sum of huge int64 values
    would overflow and could pass the capacity check)."""
    big = (1 << 63) - 1
    kw = dict(m=10, n_sink=2, n_recent=2)
    kw[which] = big
    st = lib.sig_score_topk(fake(), fake(), 1, 4, 1, 1000, kw["m"], kw["n_sink"], kw["n_recent"], fake(), 14, fake(),
                            None, fake(), 1 << 30, None)
    assert st == 1 and b"INT32_MAX" in lib.lcda_last_error()
    st = lib.sig_score_topk_w(fake(), fake(), 2, 1, 4, 1, 1000, kw["m"], kw["n_sink"], kw["n_recent"], fake(), 14,
                              fake(), None, fake(), 1 << 30, None)
    assert st == 1 and b"INT32_MAX" in lib.lcda_last_error()
    st = lib.sparse_decode_step(fake(), fake(), fake(), fake(), fake(), 0, 1, 4, 1, 128, 1000, 1, kw["m"],
                                kw["n_sink"], kw["n_recent"], fake(), 14, fake(), fake(), None, fake(), 1 << 30, None)
    assert st == 1 and b"INT32_MAX" in lib.lcda_last_error()


def test_stream_read_rejects(lib):
    """The streaming-read probe refuses null or misaligned buffers and bad grids before any launch."""
    assert lib.lcda_stream_read(None, 1 << 20, 256, fake(), 0, None) == 1
    assert lib.lcda_stream_read(fake(0x10008), 1 << 20, 256, fake(), 0, None) == 1
    assert lib.lcda_stream_read(fake(), (1 << 20) + 4, 256, fake(), 0, None) == 1
    assert lib.lcda_stream_read(fake(), 1 << 20, 0, fake(), 0, None) == 1
    assert lib.lcda_stream_read(fake(), 1 << 20, 256, None, 0, None) == 1
    assert lib.lcda_stream_read(None, 0, 256, None, 0, None) == 0   # nothing to read


def test_workspace_sizes_do_not_follow_the_knobs(lib):
    """Workspace sizes cover every accepted knob setting, so a knob changed after a workspace was sized never
    makes it too small; target-workgroup knobs beyond that range are refused."""
    shapes = [
        ("lcda_ws_bytes_cached_attn_lse", (1, 32, 8, 128, 61440, 8 * 61440 * 128)),
        ("lcda_ws_bytes_cached_attn_lse", (16, 32, 8, 128, 61440, 0)),
        ("lcda_ws_bytes_gather_attn", (8, 32, 8, 128, 4352)),
        ("lcda_ws_bytes_dense_decode_step", (1, 32, 8, 128, 61440, 8 * 61440 * 128, 256)),
        ("lcda_ws_bytes_dense_decode_step", (16, 32, 8, 128, 61440, 0, 512)),
        ("lcda_ws_bytes_sig_score_topk", (8, 32, 8, 131072)),
        ("lcda_ws_bytes_sparse_decode_step", (8, 32, 8, 128, 131072, 4352)),
        ("lcda_ws_bytes_sig_score_topk_w", (8, 32, 131072)),
    ]
    keys = {"dense_wgs": 2048, "dense_wgs_nt4": 2048, "valu_wgs": 2048, "gather_wgs": 2048, "gather_waves": 4,
            "rows_wgs": 2048, "rows_wgs_single": 2048, "rows_kernel": 0, "direct_blocks": 0, "topk_kernel": 0,
            "topk_subs": 1, "topk_wgs": 2048, "wide_chunk": 4096}
    before = [getattr(lib, f)(*a) for f, a in shapes]
    saved = {k: lib.lcda_get_tuning(k.encode()) for k in keys}
    try:
        for k, v in keys.items():
            assert lib.lcda_set_tuning(k.encode(), v) == 0, k
        after = [getattr(lib, f)(*a) for f, a in shapes]
    finally:
        for k, v in saved.items():
            assert lib.lcda_set_tuning(k.encode(), v) == 0
    assert after == before
    for k in ("dense_wgs", "dense_wgs_nt4", "valu_wgs", "gather_wgs", "rows_wgs", "rows_wgs_single"):
        assert lib.lcda_set_tuning(k.encode(), 4096) == 1
        assert lib.lcda_get_tuning(k.encode()) == saved[k]
