"""Pins of the CPU oracle to facts fixed by the slide decks and by mathematics.

Nothing here touches a GPU.  Each test checks the oracle against something
other than itself: values printed on the slides (fixtures in tests/golden/,
each with its citation), closed forms, invariants, or a special case that
reduces to a different routine.
"""
import json
import math
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rng(seed):
    return np.random.default_rng(seed)


def bf16_bits(x):
    """Round float32 values to bf16 (nearest-even) and return the bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- P-a ------
def test_4bit_example_distances_and_topk(orc):
    """HashAttention, 'A 32-bit signature makes scoring cheap': query 1011 against keys
    1011 / 1001 / 0110 gives distances 0 / 1 / 3 (scores 0, -1, -3)."""
    g = gold("hash_4bit_example.json")
    keys = np.array([[[int(s, 2) for s in g["keys"]]]], np.uint32)
    q = np.array([[int(g["query"], 2)]], np.uint32)
    idx, cnt, scores = orc.sig_score_topk(keys, q, m=3, n_sink=0, n_recent=0, want_scores=True)
    assert list(-scores[0, 0].astype(int)) == g["distances"]
    for m, expect in [(0, []), (1, [0]), (2, [0, 1]), (3, [0, 1, 2])]:
        idx, cnt, _ = orc.sig_score_topk(keys, q, m=m, n_sink=0, n_recent=0, cap=3)
        assert cnt[0, 0] == len(expect)
        assert list(idx[0, 0, :cnt[0, 0]]) == expect
        assert all(idx[0, 0, cnt[0, 0]:] == -1)


def test_popcount_uses_all_32_bits(orc):
    """Distances of single-bit and all-bit differences at every bit position."""
    q = np.array([[0]], np.uint32)
    keys = np.array([[[1 << b for b in range(32)] + [0xFFFFFFFF, 0]]], np.uint32)
    _, _, scores = orc.sig_score_topk(keys, q, m=0, n_sink=0, n_recent=0, want_scores=True)
    assert list(-scores[0, 0].astype(int)) == [1] * 32 + [32, 0]


def test_ties_go_to_the_lower_position(orc):
    """Reading of TOPK (the slides do not fix ties): among equal distances the lower position wins.
    Identical keys select the first m positions; mixed distances fill the quota from the left."""
    keys = np.full((1, 1, 10), 0xDEADBEEF, np.uint32)
    q = np.array([[0x12345678]], np.uint32)
    idx, cnt, _ = orc.sig_score_topk(keys, q, 3, 0, 0)
    assert list(idx[0, 0, :cnt[0, 0]]) == [0, 1, 2]
    # distances 1,0,1,1,0,1 -> both zeros, then the lowest-index one
    keys = np.array([[[1, 0, 2, 4, 0, 8]]], np.uint32)
    idx, cnt, _ = orc.sig_score_topk(keys, np.zeros((1, 1), np.uint32), 3, 0, 0)
    assert list(idx[0, 0, :cnt[0, 0]]) == [0, 1, 4]


# ---------------------------------------------------------------- P-c ------
@pytest.mark.parametrize("n", [1, 7, 300])
def test_identical_keys_give_mean_of_values(orc, n):
    """All keys equal: every weight is 1/n, so A = mean(V) and alpha = q.k/sqrt(d) + log n."""
    r = rng(1)
    d = 128
    q = r.standard_normal((1, 1, d)).astype(np.float32)
    kk = r.standard_normal(d).astype(np.float32)
    k = np.broadcast_to(kk, (1, 1, n, d)).copy()
    v = r.standard_normal((1, 1, n, d)).astype(np.float32)
    out, alpha = orc.dense_attn(q, k, v)
    np.testing.assert_allclose(out[0, 0], v[0, 0].astype(np.float64).mean(0), rtol=1e-12, atol=1e-13)
    s = float(np.dot(q[0, 0].astype(np.float64), kk.astype(np.float64))) / math.sqrt(d)
    assert alpha[0, 0] == pytest.approx(s + math.log(n), abs=1e-12)


def test_gqa_head_mapping_and_batch_stride(orc):
    """Query head hq reads KV head hq // G; batch b reads its own cache.  Each (b, h) cache
    has identical keys k_{b,h}, so every output is the mean of that cache's values."""
    r = rng(2)
    B, Hkv, G, n, d = 2, 3, 2, 5, 128
    Hq = Hkv * G
    keys = r.standard_normal((B, Hkv, d)).astype(np.float32)
    k = np.repeat(keys[:, :, None, :], n, axis=2)
    v = r.standard_normal((B, Hkv, n, d)).astype(np.float32)
    q = r.standard_normal((B, Hq, d)).astype(np.float32)
    out, alpha = orc.dense_attn(q, k, v)
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            np.testing.assert_allclose(out[b, hq], v[b, h].astype(np.float64).mean(0), rtol=1e-12, atol=1e-13)
            s = float(q[b, hq].astype(np.float64) @ keys[b, h].astype(np.float64)) / math.sqrt(d)
            assert alpha[b, hq] == pytest.approx(s + math.log(n), abs=1e-12)


def test_single_token_and_zero_query_and_empty(orc):
    r = rng(3)
    d = 128
    q = r.standard_normal((1, 2, d)).astype(np.float32)
    k = r.standard_normal((1, 1, 1, d)).astype(np.float32)
    v = r.standard_normal((1, 1, 1, d)).astype(np.float32)
    out, alpha = orc.dense_attn(q, k, v)
    for hq in range(2):
        np.testing.assert_array_equal(out[0, hq], v[0, 0, 0].astype(np.float64))
        s = float(q[0, hq].astype(np.float64) @ k[0, 0, 0].astype(np.float64)) / math.sqrt(d)
        assert alpha[0, hq] == pytest.approx(s, abs=1e-12)
    # q = 0: uniform weights, alpha = log n
    n = 50
    k = r.standard_normal((1, 1, n, d)).astype(np.float32)
    v = r.standard_normal((1, 1, n, d)).astype(np.float32)
    out, alpha = orc.dense_attn(np.zeros((1, 1, d), np.float32), k, v)
    np.testing.assert_allclose(out[0, 0], v[0, 0].astype(np.float64).mean(0), rtol=1e-12, atol=1e-13)
    assert alpha[0, 0] == pytest.approx(math.log(n), abs=1e-13)
    # n = 0: empty sum
    out, alpha = orc.dense_attn(q, np.zeros((1, 1, 0, d), np.float32), np.zeros((1, 1, 0, d), np.float32))
    assert np.all(out == 0) and np.all(np.isneginf(alpha))


def test_two_tokens_closed_form(orc):
    """n = 2: A = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1, alpha = s1 + log(1 + e^{s0-s1})."""
    r = rng(4)
    d = 128
    q = r.standard_normal((1, 1, d)).astype(np.float32)
    k = r.standard_normal((1, 1, 2, d)).astype(np.float32)
    v = r.standard_normal((1, 1, 2, d)).astype(np.float32)
    out, alpha = orc.dense_attn(q, k, v)
    s0, s1 = (k[0, 0].astype(np.float64) @ q[0, 0].astype(np.float64)) / math.sqrt(d)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    v64 = v[0, 0].astype(np.float64)
    np.testing.assert_allclose(out[0, 0], w0 * v64[0] + (1 - w0) * v64[1], rtol=1e-12, atol=1e-12)
    assert alpha[0, 0] == pytest.approx(s1 + math.log1p(math.exp(s0 - s1)), abs=1e-12)


def test_bf16_inputs_decode_exactly(orc):
    """bf16 bit patterns and their exact float32 expansions give identical results."""
    r = rng(5)
    B, Hq, Hkv, n, d = 2, 4, 2, 33, 128
    qb = bf16_bits(r.standard_normal((B, Hq, d)))
    kb = bf16_bits(r.standard_normal((B, Hkv, n, d)))
    vb = bf16_bits(r.standard_normal((B, Hkv, n, d)))
    o1, a1 = orc.dense_attn(qb, kb, vb)
    o2, a2 = orc.dense_attn(bits_to_f32(qb), bits_to_f32(kb), bits_to_f32(vb))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(a1, a2)
    # a few fixed patterns: 1.0, -2.0, 0.5, smallest normal, +0
    pats = np.array([0x3F80, 0xC000, 0x3F00, 0x0080, 0x0000], np.uint16)
    assert list(bits_to_f32(pats)) == [1.0, -2.0, 0.5, 2.0 ** -126, 0.0]
    one = np.zeros((1, 1, 128), np.uint16)
    one[0, 0, 0] = 0x3F80
    k = np.zeros((1, 1, 1, 128), np.uint16)
    v = np.zeros((1, 1, 1, 128), np.uint16)
    k[0, 0, 0, 0] = 0xC000  # -2
    v[0, 0, 0, :] = pats[2]  # 0.5
    out, alpha = orc.dense_attn(one, k, v)
    assert np.all(out == 0.5) and alpha[0, 0] == pytest.approx(-2.0 / math.sqrt(128), abs=1e-15)


def test_shared_document_equals_per_batch_copies(orc):
    r = rng(6)
    B, Hq, Hkv, n, d = 3, 4, 2, 40, 128
    q = r.standard_normal((B, Hq, d)).astype(np.float32)
    k = r.standard_normal((1, Hkv, n, d)).astype(np.float32)
    v = r.standard_normal((1, Hkv, n, d)).astype(np.float32)
    o1, a1 = orc.dense_attn(q, k, v)
    o2, a2 = orc.dense_attn(q, np.repeat(k, B, 0), np.repeat(v, B, 0))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(a1, a2)


# ---------------------------------------------------------------- P-d ------
def test_split_merge_is_exact(orc):
    """Nectar, 'The score makes exact local attention composable': splitting the softmax sum is
    exact.  attn([K; K_loc]) equals merge(attn(K), local), and any partition of the tokens merged
    piece by piece gives the dense result."""
    r = rng(7)
    B, Hq, Hkv, n, d = 2, 4, 2, 200, 128
    q = r.standard_normal((B, Hq, d)).astype(np.float32) * 2
    k = r.standard_normal((B, Hkv, n, d)).astype(np.float32)
    v = r.standard_normal((B, Hkv, n, d)).astype(np.float32)
    out_full, alpha_full = orc.dense_attn(q, k, v)
    # two parts: the first 150 tokens as the "cache", the rest as local tokens
    a, al = orc.dense_attn(q, k[:, :, :150], v[:, :, :150])
    mo, ma = orc.merge_local(q, a, al, k[:, :, 150:], v[:, :, 150:])
    np.testing.assert_allclose(mo, out_full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ma, alpha_full, rtol=0, atol=1e-12)
    # an arbitrary partition, merged left to right
    cuts = [0, 1, 37, 38, 120, 199, 200]
    acc, acc_alpha = orc.dense_attn(q, k[:, :, :1], v[:, :, :1])
    for lo, hi in zip(cuts[1:-1], cuts[2:]):
        acc, acc_alpha = orc.merge_local(q, acc, acc_alpha, k[:, :, lo:hi], v[:, :, lo:hi])
    np.testing.assert_allclose(acc, out_full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(acc_alpha, alpha_full, rtol=0, atol=1e-12)


def test_merge_with_ragged_local_counts_and_empty_sides(orc):
    r = rng(8)
    B, Hq, Hkv, n, d, nl = 3, 2, 1, 30, 128, 9
    q = r.standard_normal((B, Hq, d)).astype(np.float32)
    k = r.standard_normal((B, Hkv, n, d)).astype(np.float32)
    v = r.standard_normal((B, Hkv, n, d)).astype(np.float32)
    kl = r.standard_normal((B, Hkv, nl, d)).astype(np.float32)
    vl = r.standard_normal((B, Hkv, nl, d)).astype(np.float32)
    n_loc = np.array([0, 4, 9], np.int32)
    a, al = orc.dense_attn(q, k, v)
    mo, ma = orc.merge_local(q, a, al, kl, vl, n_loc)
    # item 0: no local tokens -> unchanged
    np.testing.assert_array_equal(mo[0], a[0])
    np.testing.assert_array_equal(ma[0], al[0])
    for b in (1, 2):
        full_k = np.concatenate([k[b:b + 1], kl[b:b + 1, :, :n_loc[b]]], axis=2)
        full_v = np.concatenate([v[b:b + 1], vl[b:b + 1, :, :n_loc[b]]], axis=2)
        fo, fa = orc.dense_attn(q[b:b + 1], full_k, full_v)
        np.testing.assert_allclose(mo[b], fo[0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ma[b], fa[0], atol=1e-12)
    # empty cached part (alpha = -inf): the merge is the local attention alone
    zero = np.zeros((B, Hq, d))
    ninf = np.full((B, Hq), -np.inf)
    mo, ma = orc.merge_local(q, zero, ninf, kl, vl)
    lo, la = orc.dense_attn(q, kl, vl)
    np.testing.assert_allclose(mo, lo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ma, la, atol=1e-12)
    # both empty
    mo, ma = orc.merge_local(q, zero, ninf, kl, vl, np.zeros(B, np.int32))
    assert np.all(mo == 0) and np.all(np.isneginf(ma))


# ---------------------------------------------------------------- P-e ------
def test_gate_form_equals_merge(orc):
    """Nectar Eq. (3.5): with Z_loc > 0, g = sigmoid(alpha - log Z_loc) and
    ATT = g A + (1 - g) A_loc equals the exact merge of Eq. (3.4)."""
    r = rng(9)
    B, Hq, Hkv, n, nl, d = 2, 4, 2, 64, 16, 128
    q = r.standard_normal((B, Hq, d)).astype(np.float32)
    k = r.standard_normal((B, Hkv, n, d)).astype(np.float32)
    v = r.standard_normal((B, Hkv, n, d)).astype(np.float32)
    kl = r.standard_normal((B, Hkv, nl, d)).astype(np.float32)
    vl = r.standard_normal((B, Hkv, nl, d)).astype(np.float32)
    a, al = orc.dense_attn(q, k, v)
    a_loc, log_z_loc = orc.dense_attn(q, kl, vl)     # A_loc and log Z_loc of the local tokens
    g = 1.0 / (1.0 + np.exp(-(al - log_z_loc)))
    gate = g[..., None] * a + (1 - g[..., None]) * a_loc
    mo, ma = orc.merge_local(q, a, al, kl, vl)
    np.testing.assert_allclose(mo, gate, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ma, np.logaddexp(al, log_z_loc), atol=1e-12)


# ---------------------------------------------------------------- P-f ------
def _sparse_case(seed, B=2, Hq=4, Hkv=2, n=100, d=128):
    r = rng(seed)
    q = r.standard_normal((B, Hq, d)).astype(np.float32)
    k = r.standard_normal((B, Hkv, n, d)).astype(np.float32)
    v = r.standard_normal((B, Hkv, n, d)).astype(np.float32)
    ks = r.integers(0, 2 ** 32, (B, Hkv, n), dtype=np.uint64).astype(np.uint32)
    qs = r.integers(0, 2 ** 32, (B, Hq), dtype=np.uint64).astype(np.uint32)
    return q, k, v, ks, qs


def test_full_budget_gives_dense(orc):
    """HashAttention, 'Only selection is approximate': with every position selected, o-hat = o."""
    q, k, v, ks, qs = _sparse_case(10)
    n = k.shape[2]
    dense_o, dense_a = orc.dense_attn(q, k, v)
    for m, s, rr in [(n, 0, 0), (n + 5, 3, 3), (0, 60, 40), (10, 50, 50)]:
        idx, cnt, _ = orc.sig_score_topk(ks, qs, m, s, rr)
        assert np.all(cnt == n)
        assert np.all(idx == np.arange(n)[None, None, :])
        o, a = orc.gather_attn(q, k, v, idx, cnt)
        np.testing.assert_allclose(o, dense_o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(a, dense_a, atol=1e-12)


def test_zero_budget_is_windows_only(orc):
    """m = 0 keeps only the fixed windows (initial + recent tokens, the StreamingLLM selector)."""
    q, k, v, ks, qs = _sparse_case(11)
    n, s, rr = k.shape[2], 8, 16
    idx, cnt, _ = orc.sig_score_topk(ks, qs, 0, s, rr)
    win = np.r_[0:s, n - rr:n]
    assert np.all(cnt == s + rr)
    assert np.all(idx[:, :, :s + rr] == win[None, None])
    o, a = orc.gather_attn(q, k, v, idx, cnt)
    wo, wa = orc.dense_attn(q, k[:, :, win], v[:, :, win])
    np.testing.assert_allclose(o, wo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(a, wa, atol=1e-12)


def test_gather_equals_dense_on_gathered_rows(orc):
    """GATHER-ATT over I is dense attention over the rows of I alone."""
    q, k, v, ks, qs = _sparse_case(12)
    idx, cnt, _ = orc.sig_score_topk(ks, qs, 13, 2, 3)
    o, a = orc.gather_attn(q, k, v, idx, cnt)
    B, Hq = q.shape[:2]
    G = Hq // k.shape[1]
    for b in range(B):
        for hq in range(Hq):
            sel = idx[b, hq, :cnt[b, hq]]
            ro, ra = orc.dense_attn(q[b:b + 1, hq:hq + 1], k[b:b + 1, hq // G:hq // G + 1, sel],
                                    v[b:b + 1, hq // G:hq // G + 1, sel])
            np.testing.assert_allclose(o[b, hq], ro[0, 0], rtol=1e-12, atol=1e-13)
            assert a[b, hq] == pytest.approx(ra[0, 0], abs=1e-12)


# ---------------------------------------------------------------- P-g ------
def test_gather_equals_masked_renormalised_softmax(orc):
    """NAtS-L backup 'the mask gradient includes renormalization': O = sum_j e^{A_j} M_j V_j / Z with
    Z = sum_j e^{A_j} M_j; with a 0/1 mask M = [j in I] this is GATHER-ATT."""
    q, k, v, ks, qs = _sparse_case(13)
    idx, cnt, _ = orc.sig_score_topk(ks, qs, 20, 4, 4)
    o, a = orc.gather_attn(q, k, v, idx, cnt)
    B, Hq, d = q.shape
    G = Hq // k.shape[1]
    for b in range(B):
        for hq in range(Hq):
            mask = np.zeros(k.shape[2])
            mask[idx[b, hq, :cnt[b, hq]]] = 1.0
            logits = (k[b, hq // G].astype(np.float64) @ q[b, hq].astype(np.float64)) / math.sqrt(d)
            e = np.exp(logits - logits.max()) * mask
            ref = (e @ v[b, hq // G].astype(np.float64)) / e.sum()
            np.testing.assert_allclose(o[b, hq], ref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- P-h ------
def test_alpha_gradient_matches_key_average(orc):
    """Nectar App. B, Eq. (B.1): grad_q alpha = (1/sqrt d) K^T softmax(K q / sqrt d).  Central
    differences of the oracle's alpha along random directions match it; this pins the 1/sqrt(d)
    scale and the natural logarithm."""
    r = rng(14)
    n, d = 80, 128
    k = r.standard_normal((1, 1, n, d))
    v = r.standard_normal((1, 1, n, d)).astype(np.float32)
    k32 = k.astype(np.float32)
    K = k32[0, 0].astype(np.float64)
    q0 = r.standard_normal(d)
    # keep q in float64 precision by using dyadic perturbations on a float32 grid
    q0 = q0.astype(np.float32).astype(np.float64)
    logits = K @ q0 / math.sqrt(d)
    p = np.exp(logits - logits.max())
    p /= p.sum()
    grad = K.T @ p / math.sqrt(d)
    h = 2.0 ** -10
    for _ in range(4):
        u = np.sign(r.standard_normal(d))       # +-1 directions keep q0 +- h u exact in float32
        qp = (q0 + h * u).astype(np.float32)[None, None]
        qm = (q0 - h * u).astype(np.float32)[None, None]
        _, ap = orc.dense_attn(qp, k32, v)
        _, am = orc.dense_attn(qm, k32, v)
        fd = (ap[0, 0] - am[0, 0]) / (2 * h)
        assert fd == pytest.approx(float(grad @ u), rel=1e-5, abs=1e-9)


# ---------------------------------------------------------------- P-i / P-m -
def test_low_temperature_limit_and_bounds(orc):
    """Nectar Eq. (B.2): (1/beta) log sum_j exp(beta q.k_j) -> max_j q.k_j, within log(n)/beta;
    and max_j s_j <= alpha <= max_j s_j + log n at any temperature."""
    r = rng(15)
    n, d = 64, 128
    k = r.standard_normal((1, 1, n, d)).astype(np.float32)
    v = r.standard_normal((1, 1, n, d)).astype(np.float32)
    q = r.standard_normal((1, 1, d)).astype(np.float32)
    K = k[0, 0].astype(np.float64)
    qk = K @ q[0, 0].astype(np.float64)
    prev_gap = None
    for beta in [2.0 ** e for e in range(0, 12, 2)]:
        qb = (q * np.float32(beta * math.sqrt(d)))  # s_j = beta q.k_j up to float32 rounding of q
        _, a = orc.dense_attn(qb, k, v)
        s = K @ qb[0, 0].astype(np.float64) / math.sqrt(d)
        assert s.max() - 1e-9 <= a[0, 0] <= s.max() + math.log(n) + 1e-9
        gap = a[0, 0] / beta - qk.max()
        assert -1e-6 <= gap <= math.log(n) / beta + 1e-6
        if prev_gap is not None:
            assert gap <= prev_gap + 1e-9
        prev_gap = gap
    assert prev_gap < 1e-3


def test_mass_captured_by_selection(orc):
    """exp(alpha_I - alpha) is the softmax mass of I: in (0, 1], equal to 1 when I holds all."""
    q, k, v, ks, qs = _sparse_case(16)
    _, dense_a = orc.dense_attn(q, k, v)
    for m in [0, 5, 50]:
        idx, cnt, _ = orc.sig_score_topk(ks, qs, m, 2, 2)
        _, a = orc.gather_attn(q, k, v, idx, cnt)
        mass = np.exp(a - dense_a)
        assert np.all(mass > 0) and np.all(mass <= 1 + 1e-12)
        assert np.all(mass < 1 - 1e-12)  # strictly less while positions are left out
    idx, cnt, _ = orc.sig_score_topk(ks, qs, k.shape[2], 0, 0)
    _, a = orc.gather_attn(q, k, v, idx, cnt)
    np.testing.assert_allclose(np.exp(a - dense_a), 1.0, atol=1e-12)


# ---------------------------------------------------------------- P-j ------
def test_residual_counterexample_numbers(orc):
    """HashAttention backup 'isolated contribution is not general optimality':
    a = (0.45, 0.35, 0.20), v = (1, -1, 1) gives o = 0.30; keeping only the largest contribution
    leaves error 0.15, keeping only the smallest leaves 0.10 (without renormalisation).  Embedded at
    d = 128 with q = sqrt(128) e1, k_i = ln(a_i) e1, v_i = v_i e1, so that s_i = ln a_i."""
    g = gold("residual_counterexample.json")
    a = np.array(g["weights_a"])
    vals = np.array(g["values_v"])
    d = 128
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = math.sqrt(d)
    k = np.zeros((1, 1, 3, d), np.float32)
    k[0, 0, :, 0] = np.log(a)
    v = np.zeros((1, 1, 3, d), np.float32)
    v[0, 0, :, 0] = vals
    o, alpha = orc.dense_attn(q, k, v)
    assert o[0, 0, 0] == pytest.approx(g["full_output_o"], abs=1e-6)
    assert alpha[0, 0] == pytest.approx(0.0, abs=1e-6)           # sum of a = 1
    def sel(ids):
        idx = np.array([[ids + [-1] * (3 - len(ids))]], np.int32)
        return orc.gather_attn(q, k, v, idx, np.array([[len(ids)]], np.int32))
    for ids, err in [([0], g["error_keep_largest_only"]), ([2], g["error_keep_smallest_only"])]:
        oh, ah = sel(ids)
        assert oh[0, 0, 0] == pytest.approx(1.0, abs=1e-6)           # renormalised: v_i itself
        unnorm = math.exp(ah[0, 0] - alpha[0, 0]) * oh[0, 0, 0]       # a_i v_i
        assert abs(o[0, 0, 0] - unnorm) == pytest.approx(err, abs=1e-6)
    oh, _ = sel([0, 1])
    assert oh[0, 0, 0] == pytest.approx((0.45 - 0.35) / 0.80, abs=1e-6)


# ---------------------------------------------------------------- P-k ------
def test_budget_accounting_example(orc):
    """HashAttention 'Budget accounting': n = 16,384, m = 1,024 plus up to 256 fixed positions
    means up to 1,280 reads, 7.81% of the context; |I| never exceeds it."""
    g = gold("budget_example.json")
    cap = orc.capacity(g["n"], g["m"], g["n_sink"], g["n_recent"])
    assert cap == g["max_reads"]
    assert round(100 * cap / g["n"], 2) == g["percent_of_context"]
    r = rng(17)
    ks = r.integers(0, 2 ** 32, (1, 2, g["n"]), dtype=np.uint64).astype(np.uint32)
    qs = r.integers(0, 2 ** 32, (1, 4), dtype=np.uint64).astype(np.uint32)
    idx, cnt, _ = orc.sig_score_topk(ks, qs, g["m"], g["n_sink"], g["n_recent"])
    assert np.all(cnt <= cap) and np.all(cnt >= g["m"])
    for hq in range(4):
        sel = idx[0, hq, :cnt[0, hq]]
        assert np.all(np.diff(sel) > 0)
        assert set(range(g["n_sink"])) <= set(sel.tolist())
        assert set(range(g["n"] - g["n_recent"], g["n"])) <= set(sel.tolist())


def test_cap_too_small_is_an_error(orc):
    ks = np.arange(10, dtype=np.uint32)[None, None]
    qs = np.zeros((1, 1), np.uint32)
    with pytest.raises(ValueError):
        orc.sig_score_topk(ks, qs, 5, 2, 2, cap=8)


# ---------------------------------------------------------------- P-l ------
def test_kv_storage_bytes():
    """Nectar: 2 n L H d bf16 entries; 36 layers x 8 KV heads x d=128 at 62,000 tokens is ~9.14 GB."""
    from long_context_decode_attn_amd import traffic
    g = gold("kv_storage_example.json")
    b = traffic.doc_kv_state_bytes(g["n"], g["layers"], g["kv_heads"], g["d"], g["bytes_per_entry"])
    assert b == 9_142_272_000
    assert round(b / 1e9, 2) == g["gigabytes_about"]


# ------------------------------------------------------- T_map (N2) --------
# phi(x) = ReLU(sign(R^T x)) ("HashAttention: Semantic Sparsity for Faster
# Inference", slide "A 32-bit signature makes scoring cheap", Eq. (1)) with a
# random projection R, the LSH selector of slide "Learning the codes matters
# more than merely hashing".  Component b is bit b of the code.

def test_sig_encode_axis_projection(orc):
    """R = the first 32 coordinate axes: bit b is x_b > 0 (zero gives 0)."""
    g = rng(501)
    x = g.standard_normal((40, 128)).astype(np.float32)
    x[3, :32] = 0.0
    x[4, 5] = -0.0
    R = np.zeros((128, 32), np.float32)
    R[np.arange(32), np.arange(32)] = 1.0
    want = ((x[:, :32] > 0).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(1).astype(np.uint32)
    np.testing.assert_array_equal(orc.sig_encode(x, R), want)
    assert orc.sig_encode(x[3:4], R)[0] == 0


def test_sig_encode_signed_permuted_axes_bf16(orc):
    """R[pi(b), b] = s_b (one entry per column): bit b is s_b * x_pi(b) > 0; bf16 inputs read exactly."""
    g = rng(502)
    xb = bf16_bits(g.standard_normal((33, 128)).astype(np.float32))
    xf = bits_to_f32(xb)
    pi = g.permutation(128)[:32]
    s = g.choice(np.array([-2.0, -0.5, 0.25, 3.0], np.float32), 32)
    R = np.zeros((128, 32), np.float32)
    R[pi, np.arange(32)] = s
    want = ((s[None, :] * xf[:, pi] > 0).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(1).astype(np.uint32)
    np.testing.assert_array_equal(orc.sig_encode(xb, R), want)


def test_sig_encode_matches_matmul_signs_away_from_zero(orc):
    """Against a library matmul in float64: every bit whose projection is not within 1e-9 of zero."""
    g = rng(503)
    x = g.standard_normal((300, 128)).astype(np.float32)
    R = g.standard_normal((128, 32)).astype(np.float32)
    z = x.astype(np.float64) @ R.astype(np.float64)
    got = orc.sig_encode(x, R)
    bits = ((got[:, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(bool)
    far = np.abs(z) > 1e-9
    assert far.mean() > 0.999
    np.testing.assert_array_equal(bits[far], (z > 0)[far])


def test_sig_encode_negation_and_scaling(orc):
    """Negating x complements every bit whose projection is nonzero; scaling by 4 changes nothing."""
    g = rng(504)
    x = g.standard_normal((64, 128)).astype(np.float32)
    R = g.standard_normal((128, 32)).astype(np.float32)
    c = orc.sig_encode(x, R)
    np.testing.assert_array_equal(orc.sig_encode(-x, R), ~c)
    np.testing.assert_array_equal(orc.sig_encode(4.0 * x, R), c)


def test_sig_encode_fewer_bits_and_empty(orc):
    """A projection of b < 32 columns gives b-bit codes; zero rows give an empty result."""
    g = rng(505)
    x = g.standard_normal((10, 128)).astype(np.float32)
    R = g.standard_normal((128, 32)).astype(np.float32)
    c32 = orc.sig_encode(x, R)
    c8 = orc.sig_encode(x, np.ascontiguousarray(R[:, :8]))
    np.testing.assert_array_equal(c8, c32 & 0xFF)
    assert orc.sig_encode(np.zeros((0, 128), np.float32), R).shape == (0,)


# ------------------------------------------------------ wider codes (N3) ----
def _brute_topk_w(ks, qs, m, s, r):
    """Brute force: distances from a bit-by-bit count, a stable sort on (distance, position), the first m,
    the windows, ascending."""
    B, Hkv, n, W = ks.shape
    Hq = qs.shape[1]
    G = Hq // Hkv
    out = []
    for b in range(B):
        for hq in range(Hq):
            x = ks[b, hq // G] ^ qs[b, hq][None, :]
            d = np.zeros(n, np.int64)
            for w in range(W):
                for bit in range(32):
                    d += ((x[:, w] >> np.uint32(bit)) & np.uint32(1)).astype(np.int64)
            order = sorted(range(n), key=lambda i: (d[i], i))
            chosen = set(order[:min(m, n)]) | set(range(min(s, n))) | set(range(max(n - r, 0), n))
            out.append((sorted(chosen), -d))
    return out


@pytest.mark.parametrize("W", [2, 4, 16])
def test_wide_topk_brute_force(orc, W):
    """Tiny inputs with few distinct codes (ties everywhere) against a brute-force selection."""
    g = rng(700 + W)
    B, Hq, Hkv, n = 2, 4, 2, 57
    pool = g.integers(0, 2 ** 32, (5, W), dtype=np.uint64).astype(np.uint32)
    ks = pool[g.integers(0, 5, (B, Hkv, n))]
    qs = g.integers(0, 2 ** 32, (B, Hq, W), dtype=np.uint64).astype(np.uint32)
    for m, s, r in [(10, 3, 4), (0, 2, 2), (57, 0, 0), (20, 30, 30)]:
        idx, cnt, sc = orc.sig_score_topk_w(ks, qs, m, s, r, want_scores=True)
        for row, (want, negd) in enumerate(_brute_topk_w(ks, qs, m, s, r)):
            b, hq = divmod(row, Hq)
            assert cnt[b, hq] == len(want)
            np.testing.assert_array_equal(idx[b, hq, :len(want)], want)
            assert np.all(idx[b, hq, len(want):] == -1)
            np.testing.assert_array_equal(sc[b, hq], negd)


def test_wide_topk_one_word_and_constant_words(orc):
    """W = 1 is the 32-bit selection; extra words that every key shares with the query change nothing."""
    g = rng(710)
    B, Hq, Hkv, n = 1, 4, 1, 3000
    ks = g.integers(0, 2 ** 32, (B, Hkv, n), dtype=np.uint64).astype(np.uint32)
    qs = g.integers(0, 2 ** 32, (B, Hq), dtype=np.uint64).astype(np.uint32)
    ri, rc, _ = orc.sig_score_topk(ks, qs, 100, 8, 8)
    i1, c1, _ = orc.sig_score_topk_w(ks[..., None], qs[..., None], 100, 8, 8)
    np.testing.assert_array_equal(i1, ri)
    np.testing.assert_array_equal(c1, rc)
    extra = g.integers(0, 2 ** 32, (B, Hq, 3), dtype=np.uint64).astype(np.uint32)
    extra[:] = extra[:, :1]       # one shared pattern per batch item
    ks4 = np.concatenate([ks[..., None], np.broadcast_to(extra[:, :1, None, :], (B, Hkv, n, 3))], axis=-1)
    qs4 = np.concatenate([qs[..., None], np.broadcast_to(extra[:, :1, :], (B, Hq, 3))], axis=-1)
    i4, c4, _ = orc.sig_score_topk_w(ks4, qs4, 100, 8, 8)
    np.testing.assert_array_equal(i4, ri)


def test_wide_topk_4bit_example_in_wide_codes(orc):
    """The slide's 4-bit example (distances 0, 1, 3) placed in the third word of 4-word codes."""
    ks = np.zeros((1, 1, 3, 4), np.uint32)
    qs = np.zeros((1, 1, 4), np.uint32)
    ks[0, 0, :, 2] = [0b1011, 0b1001, 0b0110]
    qs[0, 0, 2] = 0b1011
    idx, cnt, sc = orc.sig_score_topk_w(ks, qs, 2, 0, 0, want_scores=True)
    assert sc.tolist() == [[[0, -1, -3]]] and cnt[0, 0] == 2 and idx[0, 0].tolist() == [0, 1]
