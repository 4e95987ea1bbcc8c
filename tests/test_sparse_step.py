"""The fused sparse decode step (sparse_decode_step: SCORE + TOPK + GATHER-ATT in one launch) against the
CPU oracle, through the C ABI: indices and counts bit-exact (the oracle's sig_score_topk), outputs and
alphas within the dense path's tolerances (the oracle's gather_attn over the oracle's indices)."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import ops, synth
from tests.util import assert_close, sig_np, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True, params=[1, 0], ids=["fused", "two_calls"])
def sparse_form(request):
    """Both forms of the step: one launch (the fused kernel) and the two calls."""
    old = ops.get_tuning("sparse_fused")
    ops.set_tuning("sparse_fused", request.param)
    yield request.param
    ops.set_tuning("sparse_fused", old)


def _sigs(shape, seed, pool=None):
    g = np.random.default_rng(seed)
    if pool:
        vals = g.integers(0, 2 ** 32, pool, dtype=np.uint64).astype(np.uint32)
        a = vals[g.integers(0, pool, shape)]
    else:
        a = g.integers(0, 2 ** 32, shape, dtype=np.uint64).astype(np.uint32)
    return torch.from_numpy(a.view(np.int32).copy())


def _case(orc, B, Hq, Hkv, n, m, s, r, dtype, seed, shared=False, pool=None, check_rows=None):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, 128), generator=g).to(dtype)
    Bk = 1 if shared else B
    k = torch.randn((Bk, Hkv, n, 128), generator=g).to(dtype)
    v = torch.randn((Bk, Hkv, n, 128), generator=g).to(dtype)
    ks = _sigs((B, Hkv, n), seed + 1, pool)
    qs = _sigs((B, Hq), seed + 2, pool)
    print("case sparse step B=%d Hq=%d Hkv=%d n=%d m=%d s=%d r=%d %s shared=%s" % (B, Hq, Hkv, n, m, s, r, dtype,
                                                                                  shared), flush=True)
    idx, cnt, out, alpha = ops.sparse_decode_step(ks.to(DEV), qs.to(DEV), q.to(DEV), k.to(DEV), v.to(DEV), m, s, r)
    torch.cuda.synchronize()
    ri, rc, _ = orc.sig_score_topk(sig_np(ks), sig_np(qs), m, s, r)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    ro, ra = orc.gather_attn(to_np(q), to_np(k), to_np(v), ri, rc)
    assert_close(out, alpha, ro, ra, dtype, "sparse step B=%d n=%d m=%d" % (B, n, m))
    return idx, cnt, out, alpha


@pytest.mark.parametrize("B,Hq,Hkv,n,m,s,r", [
    (8, 32, 8, 32768, 1024, 128, 128),     # config 4's shape at n = 32,768: 4 parts per (b, KV head)
    (2, 8, 2, 20000, 625, 128, 128),       # 5 parts of 4,096, ragged
    (16, 32, 8, 65535, 2048, 3000, 9000),  # 2 parts of 32,768, windows spanning thread ranges
    (4, 8, 8, 40000, 1250, 16, 16),        # G = 1: 16 wavefronts per head
    (16, 24, 8, 9000, 300, 64, 64),        # G = 3: 5 wavefronts per head, one idle
    (8, 32, 8, 32768, 0, 5, 9),            # windows only
    (2, 8, 2, 3000, 3000, 0, 0),           # full budget: equals dense attention; lists read back from idx
    (1, 4, 1, 100, 10, 2, 2),              # one part, finished in place
])
def test_sparse_step_shapes(orc, B, Hq, Hkv, n, m, s, r):
    _case(orc, B, Hq, Hkv, n, m, s, r, torch.bfloat16, 700 + n % 97 + m)


def test_sparse_step_fp32_config1(orc):
    """Config 1 (fp32 rows, n = 4,096, m = 128 + 16 + 64): one part per KV head."""
    cfg = synth.CONFIGS[1]
    x = synth.make_inputs(cfg)
    idx, cnt, out, alpha = ops.sparse_decode_step(x["key_sigs"].to(DEV), x["q_sigs"].to(DEV), x["q"].to(DEV),
                                                  x["k"].to(DEV), x["v"].to(DEV), cfg.m, cfg.n_sink, cfg.n_recent)
    torch.cuda.synchronize()
    ri, rc, _ = orc.sig_score_topk(sig_np(x["key_sigs"]), sig_np(x["q_sigs"]), cfg.m, cfg.n_sink, cfg.n_recent)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    ro, ra = orc.gather_attn(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), ri, rc)
    assert_close(out, alpha, ro, ra, torch.float32, "config 1 sparse step")


def test_sparse_step_fp32_multi_part(orc):
    _case(orc, 2, 8, 2, 9001, 300, 16, 16, torch.float32, 760)


def test_sparse_step_shared_document(orc):
    _case(orc, 4, 8, 2, 12000, 400, 8, 8, torch.bfloat16, 770, shared=True)


def test_sparse_step_massive_ties(orc):
    _case(orc, 2, 8, 2, 9000, 700, 8, 8, torch.bfloat16, 780, pool=2)


def test_sparse_step_two_call_fallback(orc):
    """G = 8 is not taken by the one-launch form: the step runs as sig_score_topk then gather_attn."""
    _case(orc, 2, 16, 2, 5000, 200, 16, 16, torch.bfloat16, 790)


def test_sparse_step_exchange_fallback(orc):
    """With a zero exchange wait the workgroups count their partners' parts themselves: same results."""
    old = ops.get_tuning("topk_spin")
    ops.set_tuning("topk_spin", 0)
    try:
        _case(orc, 8, 32, 8, 32768, 1024, 128, 128, torch.bfloat16, 800)
    finally:
        ops.set_tuning("topk_spin", old)


def test_sparse_step_matches_the_two_calls():
    """Indices and counts identical to sig_score_topk's; outputs equal gather_attn's to summation order."""
    cfg = synth.CONFIGS[4]
    x = synth.make_inputs(cfg, n=32768, device=DEV)
    idx, cnt, out, alpha = ops.sparse_decode_step(x["key_sigs"], x["q_sigs"], x["q"], x["k"], x["v"], 1024, 128, 128)
    i2, c2, _ = ops.sig_score_topk(x["key_sigs"], x["q_sigs"], 1024, 128, 128)
    o2, a2 = ops.gather_attn(x["q"], x["k"], x["v"], i2, c2)
    torch.cuda.synchronize()
    assert torch.equal(idx, i2) and torch.equal(cnt, c2)
    err = (torch.linalg.vector_norm(out - o2, dim=-1) / torch.linalg.vector_norm(o2, dim=-1)).max().item()
    assert err < 1e-5, err
    assert (alpha - a2).abs().max().item() < 1e-5


def test_sparse_step_config4_full_size(orc):
    """Config 4 at full size as the benchmark runs it: every index bit-exact; outputs of sampled (batch item,
    KV head) slices against the oracle."""
    cfg = synth.CONFIGS[4]
    x = synth.make_inputs(cfg, device=DEV)
    G = cfg.Hq // cfg.Hkv
    print("case sparse step config 4 full size", flush=True)
    idx, cnt, out, alpha = ops.sparse_decode_step(x["key_sigs"], x["q_sigs"], x["q"], x["k"], x["v"], cfg.m,
                                                  cfg.n_sink, cfg.n_recent)
    torch.cuda.synchronize()
    ri, rc, _ = orc.sig_score_topk(sig_np(x["key_sigs"]), sig_np(x["q_sigs"]), cfg.m, cfg.n_sink, cfg.n_recent)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    for b, h in [(0, 0), (2, 3), (7, 7)]:
        hs = slice(h * G, (h + 1) * G)
        go, ga = orc.gather_attn(to_np(x["q"][b:b + 1, hs]), to_np(x["k"][b:b + 1, h:h + 1]),
                                 to_np(x["v"][b:b + 1, h:h + 1]), ri[b:b + 1, hs], rc[b:b + 1, hs])
        assert_close(out[b:b + 1, hs], alpha[b:b + 1, hs], go, ga, torch.bfloat16, "config 4 b=%d h=%d" % (b, h))
