"""TOPK of the oracle against a brute-force definition written independently.

Position i is in the top m iff fewer than m positions j precede it in the order
(distance ascending, position ascending); the selected set adds the first
n_sink and last n_recent positions and is listed in ascending order.  The
distance here is counted with Python's bin().count, not the oracle's bit loop,
and membership by an O(n^2) count instead of a sort.  Signatures are drawn from
a small pool so that equal distances (ties) are common.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import oracle as _o


def brute(keys, q, m, s, r):
    n = len(keys)
    dist = [bin(int(k) ^ int(q)).count("1") for k in keys]
    sel = []
    for i in range(n):
        before = sum(1 for j in range(n) if (dist[j], j) < (dist[i], i))
        if before < m or i < s or i >= n - r:
            sel.append(i)
    return sel, [-d for d in dist]


@st.composite
def cases(draw):
    n = draw(st.integers(0, 64))
    pool = draw(st.lists(st.integers(0, 2 ** 32 - 1), min_size=1, max_size=6))
    keys = draw(st.lists(st.sampled_from(pool), min_size=n, max_size=n))
    heads = draw(st.integers(1, 3))
    qs = draw(st.lists(st.integers(0, 2 ** 32 - 1), min_size=heads, max_size=heads))
    m = draw(st.integers(0, n + 3))
    s = draw(st.integers(0, n + 3))
    r = draw(st.integers(0, n + 3))
    return keys, qs, m, s, r


@settings(max_examples=400, deadline=None)
@given(cases())
def test_topk_equals_rank_count_definition(case):
    keys, qs, m, s, r = case
    orc = _o.default()
    ks = np.array(keys, np.uint32).reshape(1, 1, -1)
    qa = np.array(qs, np.uint32).reshape(1, -1)
    cap = min(len(keys), m + s + r)
    idx, cnt, scores = orc.sig_score_topk(ks, qa, m, s, r, cap=cap, want_scores=True)
    for h, qv in enumerate(qs):
        sel, sc = brute(keys, qv, m, s, r)
        assert cnt[0, h] == len(sel)
        assert list(idx[0, h, :cnt[0, h]]) == sel
        assert all(idx[0, h, cnt[0, h]:] == -1)
        assert list(scores[0, h]) == sc
