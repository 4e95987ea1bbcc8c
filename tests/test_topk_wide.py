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


@pytest.mark.parametrize("W", [1, 4, 16])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (6, 2), (24, 2), (16, 2)])
def test_wide_head_groups(orc, W, Hq, Hkv):
    """G = 1, 3, 12 and 8 query heads per KV head: one workgroup takes up to 8 of a KV head's query heads (a
    partial group when G is not 1, 2, 4 or 8); chunks and windows as in the main shape."""
    _case(orc, W, 1, Hq, Hkv, 9000, 300, 40, 70, 980 + W + Hq)


@pytest.mark.parametrize("W", [1, 2, 8])
def test_wide_long_chunks(orc, W):
    """n > 131,072 takes chunks of 8,192 positions (two compaction tiles each); a sink window over several
    chunks and a recent window that starts inside a chunk."""
    _case(orc, W, 1, 4, 2, 140001, 4000, 20000, 300, 990 + W, scores=False)


@pytest.mark.parametrize("W", [8, 16])
def test_wide_distances_past_255(orc, W):
    """Keys near the complement of the query: distances 32W - 3 .. 32W, so t >= 255 and the stored byte (the
    distance clamped to 255) must be resolved from the codes."""
    g = np.random.default_rng(995 + W)
    n = 7000
    qs = g.integers(0, 2 ** 32, (1, 2, W), dtype=np.uint64).astype(np.uint32)
    ks = np.repeat(~qs[:, :1, None, :], n, axis=2)
    for i in range(n):
        for f in g.integers(0, 32 * W, i % 4):
            ks[0, 0, i, f // 32] ^= np.uint32(1 << int(f % 32))
    ks = np.ascontiguousarray(ks)
    for m in (10, 3000, 6999):
        print("case wide topk past 255 W=%d m=%d" % (W, m), flush=True)
        kt = torch.from_numpy(ks.view(np.int32)).to(DEV)
        qt = torch.from_numpy(qs.view(np.int32)).to(DEV)
        idx, cnt, sc = ops.sig_score_topk_w(kt, qt, m, 5, 5, want_scores=True)
        torch.cuda.synchronize()
        ri, rc, rs = orc.sig_score_topk_w(ks, qs, m, 5, 5, want_scores=True)
        np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
        np.testing.assert_array_equal(idx.cpu().numpy(), ri)
        np.testing.assert_array_equal(sc.cpu().numpy(), rs)


def test_wide_one_word_matches_32bit(orc):
    """W = 1 through sig_score_topk_w and the one-word path sig_score_topk select the same positions."""
    g = np.random.default_rng(999)
    ks = g.integers(0, 2 ** 32, (2, 2, 20000), dtype=np.uint64).astype(np.uint32)
    qs = g.integers(0, 2 ** 32, (2, 8), dtype=np.uint64).astype(np.uint32)
    kt = torch.from_numpy(ks.view(np.int32)).to(DEV)
    qt = torch.from_numpy(qs.view(np.int32)).to(DEV)
    iw, cw, _ = ops.sig_score_topk_w(kt.unsqueeze(-1).contiguous(), qt.unsqueeze(-1).contiguous(), 625, 128, 128)
    i1, c1, _ = ops.sig_score_topk(kt, qt, 625, 128, 128)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cw.cpu().numpy(), c1.cpu().numpy())
    np.testing.assert_array_equal(iw.cpu().numpy(), i1.cpu().numpy())


def test_wide_many_chunks(orc):
    """n = 1,100,001: more than 32 chunks per head, so the select pass stages the chunks' histograms block by
    block (all positions first, then each block again with its window parts)."""
    _case(orc, 2, 1, 2, 1, 1100001, 30000, 40000, 5000, 1001, scores=False)


@pytest.mark.parametrize("W", [8, 16])
def test_wide_bench_shape_every_row(orc, W):
    """The shape the code-width sweep times (B = 8, Hkv = 8, Hq = 32, n = 131,072, m = n/32, 128 + 128 window
    positions; random codes): every row's indices and count, bit-exact."""
    n = 131072
    _case(orc, W, 8, 32, 8, n, n // 32, 128, 128, 1100 + W, scores=False)


@pytest.mark.parametrize("chunk", [4096, 32768])
def test_wide_chunk_knob(orc, chunk):
    """The chunk length knob at both ends of its range: 25 chunks of 4,096 positions or 4 of 32,768 (one
    workspace serves both), windows over several chunks, ragged last chunk; 1, 4 and 16 words."""
    old = ops.get_tuning("wide_chunk")
    ops.set_tuning("wide_chunk", chunk)
    try:
        for W in (1, 4, 16):
            _case(orc, W, 2, 8, 2, 100003, 3000, 9000, 5000, 1200 + W, scores=(W == 1))
    finally:
        ops.set_tuning("wide_chunk", old)
