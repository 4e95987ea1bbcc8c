"""Sparse path on the GPU (through the C ABI) against the CPU oracle.

sig_score_topk: indices, counts and scores bit-exact.
gather_attn: same tolerances as the dense path; fed the oracle's indices (kernel
isolation) and end to end."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import ops, synth
from tests.util import assert_close, sig_np, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sigs(shape, seed, pool=None):
    g = np.random.default_rng(seed)
    if pool:
        vals = g.integers(0, 2 ** 32, pool, dtype=np.uint64).astype(np.uint32)
        a = vals[g.integers(0, pool, shape)]
    else:
        a = g.integers(0, 2 ** 32, shape, dtype=np.uint64).astype(np.uint32)
    return torch.from_numpy(a.view(np.int32).copy())


def _topk_case(orc, B, Hq, Hkv, n, m, s, r, seed, pool=None, scores=True, cap=None):
    ks = _sigs((B, Hkv, n), seed, pool)
    qs = _sigs((B, Hq), seed + 1, pool)
    print("case topk B=%d Hq=%d Hkv=%d n=%d m=%d s=%d r=%d pool=%s" % (B, Hq, Hkv, n, m, s, r, pool), flush=True)
    idx, cnt, sc = ops.sig_score_topk(ks.to(DEV), qs.to(DEV), m, s, r, cap=cap, want_scores=scores)
    torch.cuda.synchronize()
    ri, rc, rs = orc.sig_score_topk(sig_np(ks), sig_np(qs), m, s, r, cap=cap, want_scores=scores)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    if scores:
        np.testing.assert_array_equal(sc.cpu().numpy(), rs)
    return ks, qs, idx, cnt


def test_four_bit_example(orc, topk_kernel):
    """HashAttention's illustrative example: query 1011 vs keys 1011 / 1001 / 0110 -> distances 0 / 1 / 3."""
    ks = torch.tensor([[[0b1011, 0b1001, 0b0110]]], dtype=torch.int32)
    qs = torch.tensor([[0b1011]], dtype=torch.int32)
    idx, cnt, sc = ops.sig_score_topk(ks.to(DEV), qs.to(DEV), 2, 0, 0, want_scores=True)
    assert sc.cpu().tolist() == [[[0, -1, -3]]]
    assert cnt.item() == 2 and idx.cpu().tolist() == [[[0, 1]]]


@pytest.mark.parametrize("n,m,s,r", [
    (1, 1, 0, 0), (5, 2, 1, 1), (100, 10, 3, 7), (100, 0, 4, 4), (100, 100, 0, 0), (100, 150, 2, 2),
    (100, 10, 60, 50), (4095, 300, 16, 64), (4096, 300, 16, 64), (4097, 300, 16, 64), (10001, 1000, 128, 128),
    (20000, 625, 0, 0), (20000, 0, 0, 0), (20000, 19000, 5, 5), (9000, 50, 4100, 20),
])
def test_topk_shapes(orc, n, m, s, r, topk_kernel):
    _topk_case(orc, 2, 8, 2, n, m, s, r, 10 + n + m)


@pytest.mark.parametrize("B,Hq,Hkv,n,m,s,r", [
    (8, 32, 8, 32768, 1024, 128, 128),       # 4 parts of 8,192 per (b, KV head), 2 dwords per thread
    (16, 32, 8, 65536, 2048, 128, 128),      # 2 parts of 32,768 (8 dwords per thread, swizzled LDS)
    (16, 32, 8, 65535, 2048, 3000, 40000),   # ragged last part, windows spanning whole parts
    (4, 32, 8, 131072, 4096, 128, 128),      # 8 parts of 16,384
    (2, 32, 8, 131071, 4096, 1, 1),          # 16 parts of 8,192, ragged
    (16, 24, 8, 40000, 1250, 64, 64),        # G = 3
    (4, 8, 8, 100000, 60000, 0, 0),          # G = 1, most positions selected
    (8, 32, 8, 32768, 32768, 0, 0),          # full budget
    (8, 32, 8, 32768, 0, 5, 9),              # windows only
])
def test_topk_unit_shapes(orc, B, Hq, Hkv, n, m, s, r):
    """The one-launch TOPK at every part size (1 to 8 dwords of distance bytes per thread and head) with
    several parts per (b, KV head) exchanging their histograms; ragged ends, windows spanning whole parts,
    G = 1 and 3, a full budget and windows only."""
    _topk_case(orc, B, Hq, Hkv, n, m, s, r, 500 + n % 101 + m, scores=n * B * Hq <= (1 << 23))


def test_topk_unit_exchange_fallback(orc):
    """With a zero wait the workgroups that do not arrive last count their partners' parts from the codes
    themselves: the same indices (the path taken when the workgroups of a launch are not all resident)."""
    old = ops.get_tuning("topk_spin")
    ops.set_tuning("topk_spin", 0)
    try:
        _topk_case(orc, 8, 32, 8, 32768, 1024, 128, 128, 611, scores=False)
        _topk_case(orc, 2, 32, 8, 131071, 4096, 300, 7000, 612, scores=False)
    finally:
        ops.set_tuning("topk_spin", old)


def test_topk_unit_skewed_parts(orc):
    """Workgroups of one (b, KV head) whose own steps would put t far apart: every fourth step of 4,096 positions
    holds near copies of the first query head's code (0 to 2 bits off), the others random codes, so the steps held
    by some workgroups take all of the top m and the others none (their own histograms alone would give t ~10).
    The other heads see random codes everywhere.  Indices bit-exact, also with a zero wait (every workgroup that
    does not arrive last counts its partners' parts itself)."""
    B, Hq, Hkv, n, m = 2, 8, 2, 131072, 4096
    G = Hq // Hkv
    g = np.random.default_rng(777)
    ks = g.integers(0, 2 ** 32, (B, Hkv, n), dtype=np.uint64).astype(np.uint32)
    qs = g.integers(0, 2 ** 32, (B, Hq), dtype=np.uint64).astype(np.uint32)
    for b in range(B):
        for h in range(Hkv):
            for s in range(0, n // 4096, 4):
                pos = np.arange(s * 4096, (s + 1) * 4096)
                flips = np.zeros(len(pos), np.uint32)
                for k in range(2):
                    bit = g.integers(0, 32, len(pos)).astype(np.uint32)
                    on = g.integers(0, 2, len(pos)).astype(bool)
                    flips ^= np.where(on, np.left_shift(np.uint32(1), bit), np.uint32(0)).astype(np.uint32)
                ks[b, h, pos] = qs[b, h * G] ^ flips
    kt = torch.from_numpy(ks.view(np.int32).copy()).to(DEV)
    qt = torch.from_numpy(qs.view(np.int32).copy()).to(DEV)
    ri, rc, _ = orc.sig_score_topk(ks, qs, m, 128, 128)
    old = ops.get_tuning("topk_spin")
    try:
        for spin in (old, 0):
            ops.set_tuning("topk_spin", spin)
            print("case topk skewed parts spin=%d" % spin, flush=True)
            idx, cnt, _ = ops.sig_score_topk(kt, qt, m, 128, 128)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
            np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    finally:
        ops.set_tuning("topk_spin", old)


@pytest.mark.parametrize("n,m,s,r", [(300001, 5000, 5000, 3000), (270000, 4096, 128, 128), (524288, 8192, 128, 128),
                                     (524288, 100, 9000, 70000)])
def test_topk_long(orc, n, m, s, r):
    """Chunks of several 4096-position sub-chunks (n > 262,144), the 64-chunk maximum, and window parts
    longer than the prefetched 512 positions."""
    _topk_case(orc, 1, 8, 2, n, m, s, r, 20 + n % 97, scores=False)


@pytest.mark.parametrize("subs", [1, 2, 8])
def test_topk_chunk_sizes(orc, subs):
    """Chunks of 1, 2 and 8 sub-chunks: ragged last chunks and sub-chunks, windows cutting chunks,
    a chunk taking only some of its ties, and heads with few distinct codes (massive ties)."""
    old = ops.get_tuning("topk_subs")
    ops.set_tuning("topk_subs", subs)
    try:
        for n, m, s, r, pool in [(50001, 1600, 128, 128, None), (70000, 3000, 5000, 9000, None),
                                 (40000, 900, 64, 64, 3), (16384, 500, 0, 0, None)]:
            _topk_case(orc, 2, 8, 2, n, m, s, r, 300 + subs + n % 11, pool=pool, scores=False)
    finally:
        ops.set_tuning("topk_subs", old)


@pytest.mark.parametrize("pool", [1, 2, 5])
def test_topk_massive_ties(orc, pool, topk_kernel):
    """Few distinct signatures: almost every position ties; the lower position must win."""
    _topk_case(orc, 1, 4, 1, 9000, 700, 8, 8, 77 + pool, pool=pool)


def test_topk_group_sizes(orc, topk_kernel):
    for G in (1, 2, 3, 5, 8):
        _topk_case(orc, 1, 2 * G, 2, 5000, 200, 16, 16, 90 + G)


def test_topk_larger_cap(orc, topk_kernel):
    ks, qs, idx, cnt = _topk_case(orc, 1, 4, 1, 3000, 100, 10, 10, 55, cap=500)
    assert np.all(idx.cpu().numpy()[..., cnt.max().item():] == -1)


def test_config1_sparse(orc):
    cfg = synth.CONFIGS[1]
    x = synth.make_inputs(cfg)
    idx, cnt, sc = ops.sig_score_topk(x["key_sigs"].to(DEV), x["q_sigs"].to(DEV), cfg.m, cfg.n_sink, cfg.n_recent,
                                      want_scores=True)
    ri, rc, rs = orc.sig_score_topk(sig_np(x["key_sigs"]), sig_np(x["q_sigs"]), cfg.m, cfg.n_sink, cfg.n_recent,
                                    want_scores=True)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(sc.cpu().numpy(), rs)
    out, alpha = ops.gather_attn(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), idx, cnt)
    ro, ra = orc.gather_attn(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), ri, rc)
    assert_close(out, alpha, ro, ra, torch.float32, "config 1 gather")


# ---------------------------------------------------------------- gather ----
def _kv(B, Hq, Hkv, n, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, 128), generator=g).to(dtype)
    k = torch.randn((B, Hkv, n, 128), generator=g).to(dtype)
    v = torch.randn((B, Hkv, n, 128), generator=g).to(dtype)
    return q, k, v


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gather_fed_oracle_indices(orc, dtype):
    B, Hq, Hkv, n = 2, 8, 2, 7000
    q, k, v = _kv(B, Hq, Hkv, n, dtype, 31)
    ks = _sigs((B, Hkv, n), 32)
    qs = _sigs((B, Hq), 33)
    ri, rc, _ = orc.sig_score_topk(sig_np(ks), sig_np(qs), 400, 20, 30)
    rc[0, 0] = 0          # an empty selected set
    rc[1, 3] = 1          # a single row
    out, alpha = ops.gather_attn(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(ri).to(DEV),
                                 torch.from_numpy(rc).to(DEV))
    ro, ra = orc.gather_attn(to_np(q), to_np(k), to_np(v), ri, rc)
    o = out.cpu().numpy()
    assert np.all(o[0, 0] == 0) and np.isneginf(alpha[0, 0].item())
    keep = np.ones((B, Hq), bool)
    keep[0, 0] = False
    assert_close(o[keep], alpha.cpu().numpy()[keep], ro[keep], ra[keep], dtype, "gather")


def test_gather_full_budget_equals_dense(orc):
    """m >= n selects every position: GATHER-ATT then equals dense attention."""
    B, Hq, Hkv, n = 2, 8, 2, 3000
    q, k, v = _kv(B, Hq, Hkv, n, torch.bfloat16, 41)
    ks = _sigs((B, Hkv, n), 42)
    qs = _sigs((B, Hq), 43)
    idx, cnt, _ = ops.sig_score_topk(ks.to(DEV), qs.to(DEV), n, 0, 0)
    go, ga = ops.gather_attn(q.to(DEV), k.to(DEV), v.to(DEV), idx, cnt)
    ro, ra = orc.dense_attn(to_np(q), to_np(k), to_np(v))
    assert_close(go, ga, ro, ra, torch.bfloat16, "gather with all positions vs dense")


def test_gather_shared_document(orc):
    B, Hq, Hkv, n = 3, 8, 2, 2000
    g = torch.Generator().manual_seed(51)
    q = torch.randn((B, Hq, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((1, Hkv, n, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((1, Hkv, n, 128), generator=g).to(torch.bfloat16)
    ks = _sigs((B, Hkv, n), 52)
    qs = _sigs((B, Hq), 53)
    ri, rc, _ = orc.sig_score_topk(sig_np(ks), sig_np(qs), 100, 8, 8)
    out, alpha = ops.gather_attn(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(ri).to(DEV),
                                 torch.from_numpy(rc).to(DEV))
    ro, ra = orc.gather_attn(to_np(q), to_np(k), to_np(v), ri, rc)
    assert_close(out, alpha, ro, ra, torch.bfloat16, "gather shared document")


def test_config4_reduced_end_to_end(orc):
    """Config 4 recipe (random-projection signatures, m = n/32 + 128 + 128) at n = 16,384, B = 2."""
    cfg = synth.CONFIGS[4]
    n = 16384
    x = synth.make_inputs(cfg, n=n, B=2)
    m = n // 32
    idx, cnt, _ = ops.sig_score_topk(x["key_sigs"].to(DEV), x["q_sigs"].to(DEV), m, 128, 128)
    ri, rc, _ = orc.sig_score_topk(sig_np(x["key_sigs"]), sig_np(x["q_sigs"]), m, 128, 128)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    out, alpha = ops.gather_attn(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), idx, cnt)
    ro, ra = orc.gather_attn(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), ri, rc)
    assert_close(out, alpha, ro, ra, torch.bfloat16, "config 4 reduced")


def test_config4_full_size(orc):
    """Config 4 at full size (n = 131,072, B = 8, m = n/32 + 128 sink + 128 recent) as the sparse128k
    benchmark runs it: indices and counts bit-exact for every query head; gather outputs of three
    sampled (batch item, KV head) slices against the oracle."""
    cfg = synth.CONFIGS[4]
    x = synth.make_inputs(cfg, device=DEV)
    G = cfg.Hq // cfg.Hkv
    print("case config 4 full size n=%d B=%d m=%d" % (cfg.n, cfg.B, cfg.m), flush=True)
    idx, cnt, _ = ops.sig_score_topk(x["key_sigs"], x["q_sigs"], cfg.m, cfg.n_sink, cfg.n_recent)
    out, alpha = ops.gather_attn(x["q"], x["k"], x["v"], idx, cnt)
    torch.cuda.synchronize()
    ri, rc, _ = orc.sig_score_topk(sig_np(x["key_sigs"]), sig_np(x["q_sigs"]), cfg.m, cfg.n_sink, cfg.n_recent)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    for b, h in [(0, 0), (3, 5), (7, 7)]:
        hs = slice(h * G, (h + 1) * G)
        go, ga = orc.gather_attn(to_np(x["q"][b:b + 1, hs]), to_np(x["k"][b:b + 1, h:h + 1]),
                                 to_np(x["v"][b:b + 1, h:h + 1]), ri[b:b + 1, hs], rc[b:b + 1, hs])
        assert_close(out[b:b + 1, hs], alpha[b:b + 1, hs], go, ga, torch.bfloat16, "config 4 b=%d h=%d" % (b, h))


def test_gather_clamps_out_of_range_entries(orc):
    """Regression: counts beyond cap (or negative) and positions outside [0, n) are clamped by the
    kernel (results for such rows are undefined, but nothing is read out of bounds); valid rows in
    the same call are unaffected."""
    B, Hq, Hkv, n, cap = 2, 8, 2, 3000, 64
    q, k, v = _kv(B, Hq, Hkv, n, torch.bfloat16, 61)
    g = np.random.default_rng(62)
    idx = g.integers(0, n, (B, Hq, cap)).astype(np.int32)
    cnt = g.integers(0, cap + 1, (B, Hq)).astype(np.int32)
    bad_idx = idx.copy()
    bad_cnt = cnt.copy()
    bad_idx[0, 1, :] = g.integers(-(1 << 30), 1 << 30, cap).astype(np.int32)
    bad_cnt[0, 2] = cap + 1000
    bad_cnt[1, 5] = -7
    out, alpha = ops.gather_attn(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(bad_idx).to(DEV),
                                 torch.from_numpy(bad_cnt).to(DEV))
    torch.cuda.synchronize()
    ro, ra = orc.gather_attn(to_np(q), to_np(k), to_np(v), idx, cnt)
    keep = np.ones((B, Hq), bool)
    keep[0, 1] = keep[0, 2] = keep[1, 5] = False
    assert_close(out.cpu().numpy()[keep], alpha.cpu().numpy()[keep], ro[keep], ra[keep], torch.bfloat16,
                 "gather rows next to clamped rows")
    assert torch.all(out[1, 5] == 0) and torch.isneginf(alpha[1, 5])     # a negative count is an empty set


@pytest.mark.parametrize("waves,wgs,variant", [(4, 2048, 0), (4, 16, 0), (8, 16, 0), (8, 512, 0), (16, 16, 0),
                                               (16, 300, 0), (4, 16, 1), (4, 512, 1)])
def test_gather_workgroup_shapes(orc, waves, wgs, variant):
    """GATHER-ATT with 4, 8 or 16 wavefronts per workgroup, as one split per row finished in place (few
    workgroups) and as several splits merged by the combine pass, with nontemporal or (variant 1, four
    wavefronts) cached row loads; an empty and a one-row set included."""
    old = (ops.get_tuning("gather_waves"), ops.get_tuning("gather_wgs"), ops.get_tuning("gather_variant"))
    ops.set_tuning("gather_waves", waves)
    ops.set_tuning("gather_wgs", wgs)
    ops.set_tuning("gather_variant", variant)
    try:
        B, Hq, Hkv, n = 2, 8, 2, 9000
        q, k, v = _kv(B, Hq, Hkv, n, torch.bfloat16, 81)
        ks = _sigs((B, Hkv, n), 82)
        qs = _sigs((B, Hq), 83)
        ri, rc, _ = orc.sig_score_topk(sig_np(ks), sig_np(qs), 700, 64, 64)
        rc[0, 1] = 0
        rc[1, 2] = 1
        print("case gather waves=%d wgs=%d variant=%d" % (waves, wgs, variant), flush=True)
        out, alpha = ops.gather_attn(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(ri).to(DEV),
                                     torch.from_numpy(rc).to(DEV))
        torch.cuda.synchronize()
        ro, ra = orc.gather_attn(to_np(q), to_np(k), to_np(v), ri, rc)
        keep = np.ones((B, Hq), bool)
        keep[0, 1] = False
        assert_close(out.cpu().numpy()[keep], alpha.cpu().numpy()[keep], ro[keep], ra[keep], torch.bfloat16,
                     "gather waves=%d wgs=%d" % (waves, wgs))
        assert torch.all(out[0, 1] == 0) and torch.isneginf(alpha[0, 1])
    finally:
        ops.set_tuning("gather_waves", old[0])
        ops.set_tuning("gather_wgs", old[1])
        ops.set_tuning("gather_variant", old[2])
