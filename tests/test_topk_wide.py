"""SCORE + TOPK over codes of W 32-bit words (64 to 512 bits) on the GPU against the oracle: indices, counts and
scores bit-exact ("HashAttention: Semantic Sparsity for Faster Inference", slide "A 32-bit signature makes
scoring cheap", Eq. (2), summed over the words; the code widths of its Table 6 sweep)."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _codes(shape, seed, pool=None):
    g = np.random.default_rng(seed)
    if pool:
        vals = g.integers(0, 2 ** 32, (pool, shape[-1]), dtype=np.uint64).astype(np.uint32)
        a = vals[g.integers(0, pool, shape[:-1])]
    else:
        a = g.integers(0, 2 ** 32, shape, dtype=np.uint64).astype(np.uint32)
    return np.ascontiguousarray(a)


def _case(orc, W, B, Hq, Hkv, n, m, s, r, seed, pool=None, scores=True):
    ks = _codes((B, Hkv, n, W), seed, pool)
    qs = _codes((B, Hq, W), seed + 1, pool)
    print("case wide topk W=%d B=%d Hq=%d Hkv=%d n=%d m=%d s=%d r=%d pool=%s" % (W, B, Hq, Hkv, n, m, s, r, pool),
          flush=True)
    kt = torch.from_numpy(ks.view(np.int32)).to(DEV)
    qt = torch.from_numpy(qs.view(np.int32)).to(DEV)
    idx, cnt, sc = ops.sig_score_topk_w(kt, qt, m, s, r, want_scores=scores)
    torch.cuda.synchronize()
    ri, rc, rs = orc.sig_score_topk_w(ks, qs, m, s, r, want_scores=scores)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    if scores:
        np.testing.assert_array_equal(sc.cpu().numpy(), rs)


@pytest.mark.parametrize("W", [1, 2, 4, 8, 16])
def test_wide_shapes(orc, W):
    for n, m, s, r in [(1, 1, 0, 0), (100, 10, 3, 7), (4095, 300, 16, 64), (4097, 300, 16, 64), (20000, 625, 128, 128),
                       (9000, 50, 4100, 20), (3000, 3000, 0, 0), (5000, 0, 4, 4)]:
        _case(orc, W, 2, 8, 2, n, m, s, r, 900 + W + n)


@pytest.mark.parametrize("W,pool", [(2, 1), (4, 3), (16, 2)])
def test_wide_massive_ties(orc, W, pool):
    _case(orc, W, 1, 4, 1, 9000, 700, 8, 8, 950 + W, pool=pool)


def test_wide_large_and_empty(orc):
    _case(orc, 8, 1, 8, 2, 131072, 4096, 128, 128, 970, scores=False)
    _case(orc, 4, 2, 4, 1, 0, 10, 2, 2, 971)
