"""The T_map stage on the GPU against the oracle: random-projection codes of rows of 128 values
("HashAttention: Semantic Sparsity for Faster Inference", slide "A 32-bit signature makes scoring cheap",
Eq. (1), with the random projection of slide "Learning the codes matters more than merely hashing").

Codes are bit-exact, projections near zero included (both sides run the same fma chain in double).  Also:
appending new keys' codes into a cache's code array, and sig_score_topk_q, the scan that encodes its
queries at its head, against the oracle's encode-then-select."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import ops, synth
from tests.util import sig_np, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _proj(bits, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((128, bits), generator=g, dtype=torch.float32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,bits", [(1, 32), (2, 32), (3, 32), (7, 8), (1000, 32), (4097, 1), (513, 31)])
def test_encode_rows(orc, dtype, rows, bits):
    g = torch.Generator().manual_seed(600 + rows + bits)
    x = torch.randn((rows, 128), generator=g).to(dtype)
    R = _proj(bits, 601 + bits)
    print("case encode rows=%d bits=%d %s" % (rows, bits, dtype), flush=True)
    got = ops.sig_encode(x.to(DEV), R.to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sig_np(got), orc.sig_encode(to_np(x), R.numpy()))


def test_encode_near_zero_projections(orc):
    """Rows built so that many projections are exactly zero or within rounding of it."""
    g = torch.Generator().manual_seed(610)
    R = _proj(32, 611)
    x = torch.zeros((64, 128))
    x[1:16, :] = torch.randn((15, 128), generator=g)
    # a row orthogonal to column 0 of R up to rounding: subtract its projection
    r0 = R[:, 0].double()
    for i in range(16, 64):
        v = torch.randn(128, generator=g, dtype=torch.float64)
        v = v - (v @ r0) / (r0 @ r0) * r0
        x[i] = v.float()
    x[5, :] = 0.0
    print("case encode near-zero projections", flush=True)
    got = ops.sig_encode(x.to(DEV), R.to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sig_np(got), orc.sig_encode(x.numpy(), R.numpy()))
    assert sig_np(got)[0] == 0 and sig_np(got)[5] == 0


def test_append_key_codes_into_cache_layout(orc):
    """New keys at positions n_old .. n_old + r of a [B, Hkv, n_cap, 128] cache: their codes land at the same
    positions of a [B, Hkv, n] code array; every other code is untouched."""
    B, Hkv, n_cap, n, n_old, r = 2, 8, 300, 260, 200, 37
    g = torch.Generator().manual_seed(620)
    K = torch.randn((B, Hkv, n_cap, 128), generator=g).to(torch.bfloat16).to(DEV)
    R = _proj(32, 621).to(DEV)
    codes = torch.full((B, Hkv, n), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    print("case append key codes", flush=True)
    ops.sig_encode(K[:, :, n_old:n_old + r], R, codes=codes[:, :, n_old:n_old + r])
    torch.cuda.synchronize()
    c = sig_np(codes)
    want = orc.sig_encode(to_np(K[:, :, n_old:n_old + r].contiguous()), R.cpu().numpy())
    np.testing.assert_array_equal(c[:, :, n_old:n_old + r], want)
    assert np.all(c[:, :, :n_old] == 0x5A5A5A5A) and np.all(c[:, :, n_old + r:] == 0x5A5A5A5A)


@pytest.mark.parametrize("B,Hq,Hkv,n,m,s,r,dtype,bits", [
    (2, 32, 8, 20000, 625, 128, 128, torch.bfloat16, 32),
    (1, 8, 8, 9001, 300, 16, 16, torch.float32, 32),
    (3, 6, 2, 5000, 200, 0, 0, torch.bfloat16, 24),
    (1, 16, 2, 70000, 3000, 5000, 9000, torch.bfloat16, 32),
    (2, 8, 2, 0, 10, 2, 2, torch.bfloat16, 32),
])
def test_topk_with_encoded_queries(orc, B, Hq, Hkv, n, m, s, r, dtype, bits, topk_kernel):
    """Indices, counts and the returned query codes bit-exact against the oracle's encode + select, and the
    same indices as the unfused GPU calls."""
    g = torch.Generator().manual_seed(630 + n + Hq)
    q = torch.randn((B, Hq, 128), generator=g).to(dtype)
    R = _proj(bits, 631)
    ks = torch.randint(-(1 << 31), 1 << 31, (B, Hkv, n), generator=g, dtype=torch.int64).to(torch.int32)
    print("case topk_q B=%d Hq=%d Hkv=%d n=%d bits=%d %s" % (B, Hq, Hkv, n, bits, dtype), flush=True)
    idx, cnt, _, qs = ops.sig_score_topk_q(ks.to(DEV), q.to(DEV), R.to(DEV), m, s, r)
    torch.cuda.synchronize()
    rqs = orc.sig_encode(to_np(q), R.numpy())
    np.testing.assert_array_equal(sig_np(qs), rqs)
    ri, rc, _ = orc.sig_score_topk(sig_np(ks), rqs, m, s, r)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    qs2 = ops.sig_encode(q.to(DEV), R.to(DEV))
    idx2, cnt2, _ = ops.sig_score_topk(ks.to(DEV), qs2.reshape(B, Hq), m, s, r)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)


def test_config4_reduced_from_queries(orc):
    """Config 4's recipe with the query codes encoded on the GPU from the same projection."""
    cfg = synth.CONFIGS[4]
    x = synth.make_inputs(cfg, n=16384, B=2)
    R = synth.projection(128, 32, cfg.cid).float()
    m = 16384 // 32
    print("case config 4 reduced, encoded queries", flush=True)
    idx, cnt, _, qs = ops.sig_score_topk_q(x["key_sigs"].to(DEV), x["q"].to(DEV), R.to(DEV), m, 128, 128)
    torch.cuda.synchronize()
    rqs = orc.sig_encode(to_np(x["q"]), R.numpy())
    np.testing.assert_array_equal(sig_np(qs), rqs)
    ri, rc, _ = orc.sig_score_topk(sig_np(x["key_sigs"]), rqs, m, 128, 128)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)


# Many rows (16,384 and more) take the blocked path: persistent workgroups, a lane owning 8 rows x 8 bits.
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,bits", [(16384, 32), (16805, 32), (40000, 13), (70001, 32), (20000, 1)])
def test_encode_many_rows(orc, dtype, rows, bits):
    g = torch.Generator().manual_seed(700 + rows + bits)
    x = torch.randn((rows, 128), generator=g).to(dtype)
    R = _proj(bits, 701 + bits)
    print("case encode many rows=%d bits=%d %s" % (rows, bits, dtype), flush=True)
    got = ops.sig_encode(x.to(DEV), R.to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sig_np(got), orc.sig_encode(to_np(x), R.numpy()))


def test_encode_many_near_zero_projections(orc):
    """The blocked path on rows built so that every projection of a row lands within rounding of zero, plus
    all-zero rows: the sign of each chain's sum decides, bit for bit."""
    rows = 20000
    rng = np.random.default_rng(710)
    R = _proj(32, 711)
    v = rng.standard_normal((rows, 128))
    Rd = R.double().numpy()
    b = np.arange(rows) % 32
    rb = Rd[:, b].T                                   # the column each row is made orthogonal to
    v -= ((v * rb).sum(1) / (rb * rb).sum(1))[:, None] * rb
    x = torch.from_numpy(v.astype(np.float32))
    x[::97] = 0.0
    print("case encode many near-zero projections", flush=True)
    got = ops.sig_encode(x.to(DEV), R.to(DEV))
    torch.cuda.synchronize()
    want = orc.sig_encode(x.numpy(), R.numpy())
    np.testing.assert_array_equal(sig_np(got), want)
    assert np.all(sig_np(got)[::97] == 0)


@pytest.mark.parametrize("B,Hkv,n_cap,n,n_old,r,dtype", [
    (2, 8, 3000, 2800, 1100, 1500, torch.bfloat16),   # 1,500 rows per head: a 256-row turn straddles heads
    (8, 64, 300, 260, 200, 37, torch.bfloat16),       # 37 rows per head: a turn spans seven or eight heads
    (4, 8, 1200, 1100, 500, 600, torch.float32),
    (64, 256, 3, 2, 1, 1, torch.bfloat16),            # one new key in each of 16,384 heads
])
def test_encode_many_into_cache_layout(orc, B, Hkv, n_cap, n, n_old, r, dtype):
    """16,384 or more new keys of a [B, Hkv, n_cap, 128] cache encoded into the matching positions of a
    [B, Hkv, n] code array; every other code is untouched."""
    g = torch.Generator().manual_seed(720 + r)
    K = torch.randn((B, Hkv, n_cap, 128), generator=g).to(dtype).to(DEV)
    R = _proj(32, 721).to(DEV)
    codes = torch.full((B, Hkv, n), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    assert B * Hkv * r >= 16384
    print("case encode many into cache layout B=%d Hkv=%d r=%d %s" % (B, Hkv, r, dtype), flush=True)
    ops.sig_encode(K[:, :, n_old:n_old + r], R, codes=codes[:, :, n_old:n_old + r])
    torch.cuda.synchronize()
    c = sig_np(codes)
    want = orc.sig_encode(to_np(K[:, :, n_old:n_old + r].contiguous()), R.cpu().numpy())
    np.testing.assert_array_equal(c[:, :, n_old:n_old + r], want)
    assert np.all(c[:, :, :n_old] == 0x5A5A5A5A) and np.all(c[:, :, n_old + r:] == 0x5A5A5A5A)


def test_encode_whole_cache_sampled(orc):
    """A whole cache of 8 x 8 heads x 131,072 positions (8.4 M rows, bf16), the timed whole-cache encode's
    shape; 8,192 sampled rows and the last row against the oracle."""
    B, Hkv, n = 8, 8, 131072
    gen = torch.Generator(device=DEV).manual_seed(730)
    K = torch.randn((B, Hkv, n, 128), generator=gen, device=DEV, dtype=torch.bfloat16)
    R = _proj(32, 731).to(DEV)
    print("case encode whole cache %dx%dx%d" % (B, Hkv, n), flush=True)
    codes = ops.sig_encode(K, R)
    torch.cuda.synchronize()
    rows = B * Hkv * n
    pick = np.random.default_rng(732).choice(rows, 8192, replace=False)
    pick = np.append(pick, rows - 1)
    pt = torch.from_numpy(pick).to(DEV)
    want = orc.sig_encode(to_np(K.reshape(rows, 128)[pt]), R.cpu().numpy())
    np.testing.assert_array_equal(sig_np(codes.reshape(rows)[pt]), want)
    del K
