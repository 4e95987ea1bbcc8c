"""Planted needles (n = 524,288, B = 4, m = n/64 plus 128 sink and 128 recent positions): the sparse
step (sig_score_topk + gather_attn) and the dense one (cached_attn_lse) on the same inputs.

Against the oracle: indices and counts bit-exact, outputs within the bf16 tolerances.  Beyond parity,
the properties that make the comparison meaningful: the selected set is a subset of all positions, so
alpha over it never exceeds the dense alpha (mass captured e^{alpha_I - alpha} <= 1); the needles,
planted along the first query head of each KV group, are found; the sparse output's error against the
dense one is the one the oracle computes for the same sets."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import ops, synth
from tests.util import TOL, assert_close, sig_np, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
CFG = synth.CONFIGS[5]


def _recall(idx, cnt, pos, G):
    B, Hq = cnt.shape
    r = np.empty((B, Hq))
    for b in range(B):
        for hq in range(Hq):
            r[b, hq] = np.isin(pos[b, hq // G], idx[b, hq, :cnt[b, hq]]).mean()
    return r


def _run(x, m):
    """Sparse and dense results of one input set, all on the GPU."""
    idx, cnt, _ = ops.sig_score_topk(x["key_sigs"], x["q_sigs"], m, CFG.n_sink, CFG.n_recent)
    so, sa = ops.gather_attn(x["q"], x["k"], x["v"], idx, cnt)
    do, da = ops.cached_attn_lse(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    return idx, cnt, so, sa, do, da


def _row_err(a, b):
    return np.linalg.norm(a - b, axis=-1) / np.linalg.norm(b, axis=-1)


def test_needles_reduced(orc):
    """n = 65,536, B = 2 (m = n/64): every output checked against the oracle."""
    n, B = 65536, 2
    G = CFG.Hq // CFG.Hkv
    m = n // 64
    print("case needles reduced n=%d B=%d m=%d" % (n, B, m), flush=True)
    x = synth.make_inputs(CFG, device=DEV, n=n, B=B)
    idx, cnt, so, sa, do, da = _run(x, m)
    q, k, v = to_np(x["q"]), to_np(x["k"]), to_np(x["v"])
    ri, rc, _ = orc.sig_score_topk(sig_np(x["key_sigs"]), sig_np(x["q_sigs"]), m, CFG.n_sink, CFG.n_recent)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    ro, ra = orc.gather_attn(q, k, v, ri, rc)
    assert_close(so, sa, ro, ra, torch.bfloat16, "needles sparse")
    dro, dra = orc.dense_attn(q, k, v)
    assert_close(do, da, dro, dra, torch.bfloat16, "needles dense")

    # alpha over a subset of positions is at most the dense alpha
    assert np.all(ra <= dra + 1e-12)
    assert np.all(sa.cpu().numpy() <= da.cpu().numpy() + TOL[torch.bfloat16][1])
    rec = _recall(ri, rc, x["needle_pos"].cpu().numpy(), G)
    assert rec[:, ::G].min() >= 0.95, "needles planted along head 0 of each group are selected"
    err = _row_err(so.cpu().numpy().astype(np.float64), do.cpu().numpy().astype(np.float64))
    err_orc = _row_err(ro, dro)
    assert np.max(np.abs(err - err_orc)) <= 2 * TOL[torch.bfloat16][0]


def test_needles_full_size(orc):
    """The full shape (n = 524,288, B = 4, m = 8,192): indices bit-exact for every head; outputs of the
    sparse and dense calls checked on four sampled (batch item, KV head) slices."""
    G = CFG.Hq // CFG.Hkv
    print("case needles full size n=%d B=%d m=%d" % (CFG.n, CFG.B, CFG.m), flush=True)
    x = synth.make_inputs(CFG, device=DEV)
    idx, cnt, so, sa, do, da = _run(x, CFG.m)
    ri, rc, _ = orc.sig_score_topk(sig_np(x["key_sigs"]), sig_np(x["q_sigs"]), CFG.m, CFG.n_sink, CFG.n_recent)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    assert np.all(sa.cpu().numpy() <= da.cpu().numpy() + TOL[torch.bfloat16][1])
    rec = _recall(ri, rc, x["needle_pos"].cpu().numpy(), G)
    assert rec[:, ::G].min() >= 0.95
    for b, h in [(0, 0), (1, 7), (2, 3), (3, 5)]:
        hs = slice(h * G, (h + 1) * G)
        q = to_np(x["q"][b:b + 1, hs])
        k = to_np(x["k"][b:b + 1, h:h + 1])
        v = to_np(x["v"][b:b + 1, h:h + 1])
        go, ga = orc.gather_attn(q, k, v, ri[b:b + 1, hs], rc[b:b + 1, hs])
        assert_close(so[b:b + 1, hs], sa[b:b + 1, hs], go, ga, torch.bfloat16, "sparse b=%d h=%d" % (b, h))
        fo, fa = orc.dense_attn(q, k, v)
        assert_close(do[b:b + 1, hs], da[b:b + 1, hs], fo, fa, torch.bfloat16, "dense b=%d h=%d" % (b, h))
