"""The benchmark's algorithmic byte counts, against sums written out by hand for the workloads' shapes.

Each count is what the step must move: cached K and V rows, local K and V rows, queries, outputs, and on
the sparse path the key codes, the unique selected rows and the index lists.  Workspace partials are not
counted."""
import numpy as np

from long_context_decode_attn_amd import traffic


def test_dense_layer_fused_and_two_call():
    # 8 KV heads x 61,440 tokens x 128 x bf16, K and V; 256 local tokens per KV head; 32 query heads.
    kv = 2 * 8 * 61440 * 128 * 2              # 251,658,240
    loc = 2 * 8 * 256 * 128 * 2               # 1,048,576
    q = 32 * 128 * 2
    out = 32 * 129 * 4                        # out and alpha, fp32
    assert kv == 251658240 and loc == 1048576
    fused = traffic.dense_step_bytes(1, 32, 8, 128, 61440, 2, False, 256, fused=True)
    assert fused == kv + loc + q + out == 252731520
    # the two-call form also writes A and alpha, then reads them and q again
    two = traffic.dense_step_bytes(1, 32, 8, 128, 61440, 2, False, 256)
    assert two == fused + out + (out + q)
    # no local tokens: the document pass alone
    assert traffic.dense_step_bytes(1, 32, 8, 128, 61440, 2) == kv + q + out


def test_shared_document_layer():
    # one document read by 16 queries (K/V counted once), 512 private local tokens each
    kv = 2 * 1 * 8 * 61440 * 128 * 2
    loc = 2 * 8 * (16 * 512) * 128 * 2        # 33,554,432
    q = 16 * 32 * 128 * 2
    out = 16 * 32 * 129 * 4
    got = traffic.dense_step_bytes(16, 32, 8, 128, 61440, 2, True, 16 * 512, fused=True)
    assert got == kv + loc + q + out == 285607936
    # 36 layers of the document state: 9,059,696,640 B
    assert 36 * kv == traffic.doc_kv_state_bytes(61440, 36, 8, 128) == 9059696640


def test_unique_rows_counts_shared_positions_once():
    # B = 2, 4 query heads in groups of G = 2 (KV heads 0 and 1); padded lists with counts
    idx = np.full((2, 4, 5), -1, dtype=np.int32)
    cnt = np.zeros((2, 4), dtype=np.int32)
    lists = {(0, 0): [1, 3, 5], (0, 1): [3, 5, 7, 9], (0, 2): [0], (0, 3): [],
             (1, 0): [2, 4], (1, 1): [2, 4], (1, 2): [8, 9, 10, 11, 12], (1, 3): [12]}
    for (b, h), v in lists.items():
        idx[b, h, :len(v)] = v
        cnt[b, h] = len(v)
    # (b0, kv0): {1,3,5,7,9} = 5; (b0, kv1): {0} = 1; (b1, kv0): {2,4} = 2; (b1, kv1): {8..12} = 5
    assert traffic.unique_rows(idx, cnt, 2) == 13
    # entries past the count are not rows
    idx[0, 3, :] = 99
    assert traffic.unique_rows(idx, cnt, 2) == 13


def test_sparse_step():
    B, Hq, Hkv, d, n, cap = 8, 32, 8, 128, 131072, 4352
    uniq = 1013524
    got = traffic.sparse_step_bytes(B, Hq, Hkv, d, n, 2, cap, uniq)
    codes = B * Hkv * n * 4 + B * Hq * 4      # key codes, query codes
    rows = uniq * 2 * d * 2                   # K and V row of each unique (b, KV head, position)
    idx = 2 * B * Hq * (cap + 1) * 4          # index lists and counts, written then read
    assert got == codes + rows + idx + B * Hq * d * 2 + B * Hq * (d + 1) * 4
