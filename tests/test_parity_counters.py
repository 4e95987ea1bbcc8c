"""The split pass's in-kernel combine: the last workgroup of each unit merges the unit's rows, found
through per-unit arrival counters in the caller's workspace (each tagged with a hash of its address
and left at a zero count by every call).

Checks that results do not depend on what the workspace held before (zeros, all ones or random bytes
that must be recognised as untagged, an earlier call of another shape, the same call replayed from a
HIP graph), against the CPU oracle and, for replays, bit for bit against the eager call."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import ops
from tests.util import assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _kv(B, Hq, Hkv, n, seed, n_loc=0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((B, Hkv, n, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, Hkv, n, 128), generator=g).to(torch.bfloat16)
    kl = torch.randn((B, Hkv, n_loc, 128), generator=g).to(torch.bfloat16)
    vl = torch.randn((B, Hkv, n_loc, 128), generator=g).to(torch.bfloat16)
    return q, k, v, kl, vl


@pytest.mark.parametrize("fill", ["zeros", "ones", "random"])
def test_garbage_workspace(orc, fill):
    """Whatever bytes the workspace starts with, the counters start from zero for a new call."""
    B, Hq, Hkv, n, nl = 2, 32, 8, 8192, 100
    q, k, v, kl, vl = _kv(B, Hq, Hkv, n, 71, nl)
    nb = ops.ws_bytes_dense_decode_step(B, Hq, Hkv, 128, n, Hkv * n * 128, nl)
    if fill == "zeros":
        ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    elif fill == "ones":
        ws = torch.full((nb,), 255, dtype=torch.uint8, device=DEV)
    else:
        ws = torch.randint(0, 256, (nb,), dtype=torch.uint8, generator=torch.Generator().manual_seed(72)).to(DEV)
    print("case garbage workspace fill=%s" % fill, flush=True)
    a, al = ops.cached_attn_lse(q.to(DEV), k.to(DEV), v.to(DEV), ws=ws)
    out, alpha = ops.dense_decode_step(q.to(DEV), k.to(DEV), v.to(DEV), kl.to(DEV), vl.to(DEV), ws=ws)
    torch.cuda.synchronize()
    ro, ra = orc.dense_attn(to_np(q), to_np(k), to_np(v))
    assert_close(a, al, ro, ra, torch.bfloat16, "cached part, %s workspace" % fill)
    mo, ma = orc.merge_local(to_np(q), ro, ra, to_np(kl), to_np(vl), np.full(B, nl, np.int32))
    assert_close(out, alpha, mo, ma, torch.bfloat16, "fused step, %s workspace" % fill)


@pytest.mark.parametrize("fill", ["ones", "random"])
def test_garbage_workspace_gather_and_fp32(orc, fill):
    """The vector-ALU split (GATHER-ATT, and the fp32 dense path) with its combine pass on a workspace of
    garbage; each call runs twice on one workspace."""
    B, Hq, Hkv, n, cap = 2, 16, 4, 6000, 1500
    q, k, v, _, _ = _kv(B, Hq, Hkv, n, 73)
    g = np.random.default_rng(74)
    idx = np.full((B, Hq, cap), -1, np.int32)
    cnt = g.integers(0, cap + 1, (B, Hq)).astype(np.int32)
    cnt[0, 0] = 0
    for b in range(B):
        for h in range(Hq):
            idx[b, h, :cnt[b, h]] = np.sort(g.choice(n, cnt[b, h], replace=False))
    nb = max(ops.ws_bytes_gather_attn(B, Hq, Hkv, 128, cap), ops.ws_bytes_cached_attn_lse(B, Hq, Hkv, 128, n, Hkv * n * 128))
    if fill == "ones":
        ws = torch.full((nb,), 255, dtype=torch.uint8, device=DEV)
    else:
        ws = torch.randint(0, 256, (nb,), dtype=torch.uint8, generator=torch.Generator().manual_seed(75)).to(DEV)
    print("case garbage workspace (gather, fp32) fill=%s" % fill, flush=True)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    it, ct = torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV)
    res = [ops.gather_attn(qd, kd, vd, it, ct, ws=ws) for _ in range(2)]
    q32, k32, v32 = q.float(), k.float(), v.float()
    res32 = [ops.cached_attn_lse(q32.to(DEV), k32.to(DEV), v32.to(DEV), ws=ws) for _ in range(2)]
    torch.cuda.synchronize()
    ro, ra = orc.gather_attn(to_np(q), to_np(k), to_np(v), idx, cnt)
    for o, a in res:
        assert_close(o, a, ro, ra, torch.bfloat16, "gather, %s workspace" % fill)
    ro, ra = orc.dense_attn(to_np(q32), to_np(k32), to_np(v32))
    for o, a in res32:
        assert_close(o, a, ro, ra, torch.float32, "fp32 dense, %s workspace" % fill)


@pytest.mark.parametrize("fill", ["ones", "random"])
def test_garbage_workspace_topk(orc, fill):
    """TOPK: histogram rows of earlier calls (and of window parts no chunk has) left in the workspace are
    never read; indices stay bit-exact whatever the workspace held, over repeated calls of two shapes."""
    g = np.random.default_rng(76)
    cases = [(2, 8, 2, 40000, 1300, 64, 64), (3, 4, 1, 9001, 300, 16, 16)]
    nb = max(ops.ws_bytes_sig_score_topk(B, Hq, Hkv, n) for B, Hq, Hkv, n, _, _, _ in cases)
    if fill == "ones":
        ws = torch.full((nb,), 255, dtype=torch.uint8, device=DEV)
    else:
        ws = torch.randint(0, 256, (nb,), dtype=torch.uint8, generator=torch.Generator().manual_seed(77)).to(DEV)
    print("case garbage workspace (topk) fill=%s" % fill, flush=True)
    for rep in range(2):
        for B, Hq, Hkv, n, m, s_, r_ in cases:
            ks = g.integers(0, 2 ** 32, (B, Hkv, n), dtype=np.uint64).astype(np.uint32)
            qs = g.integers(0, 2 ** 32, (B, Hq), dtype=np.uint64).astype(np.uint32)
            kt = torch.from_numpy(ks.view(np.int32).copy()).to(DEV)
            qt = torch.from_numpy(qs.view(np.int32).copy()).to(DEV)
            idx, cnt, _ = ops.sig_score_topk(kt, qt, m, s_, r_, ws=ws)
            torch.cuda.synchronize()
            ri, rc, _ = orc.sig_score_topk(ks, qs, m, s_, r_)
            np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
            np.testing.assert_array_equal(idx.cpu().numpy(), ri)


def test_one_workspace_many_calls(orc):
    """Calls of different shapes back to back on one workspace (counters of one call left for the next)."""
    ws = torch.empty(1 << 24, dtype=torch.uint8, device=DEV)
    cases = [(1, 32, 8, 20000), (2, 8, 2, 3001), (1, 32, 8, 61440 // 4), (3, 16, 4, 777)]
    outs = []
    for i in range(3):
        for B, Hq, Hkv, n in cases:
            q, k, v, _, _ = _kv(B, Hq, Hkv, n, 80 + n)
            assert ops.ws_bytes_cached_attn_lse(B, Hq, Hkv, 128, n, Hkv * n * 128) <= ws.numel()
            outs.append((q, k, v) + ops.cached_attn_lse(q.to(DEV), k.to(DEV), v.to(DEV), ws=ws))
    torch.cuda.synchronize()
    print("case one workspace, %d calls" % len(outs), flush=True)
    for q, k, v, a, al in outs[-len(cases):]:
        ro, ra = orc.dense_attn(to_np(q), to_np(k), to_np(v))
        assert_close(a, al, ro, ra, torch.bfloat16, "call on a shared workspace")
    for (q, k, v, a, al), (_, _, _, a2, al2) in zip(outs[:len(cases)], outs[-len(cases):]):
        assert torch.equal(a, a2) and torch.equal(al, al2)


def test_graph_replays_match_eager():
    """A captured decode step replays with the same counter tag; eager calls on the same workspace run in
    between.  Every replay equals an eager call on the same inputs, bit for bit."""
    B, Hq, Hkv, n, nl = 1, 32, 8, 16384, 256
    q, k, v, kl, vl = (t.to(DEV) for t in _kv(B, Hq, Hkv, n, 90, nl))
    nb = ops.ws_bytes_dense_decode_step(B, Hq, Hkv, 128, n, Hkv * n * 128, nl)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    ws_ref = torch.empty(nb, dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, 128), device=DEV)
    alpha = torch.empty((B, Hq), device=DEV)
    ref_o = torch.empty_like(out)
    ref_a = torch.empty_like(alpha)

    def step():
        ops.dense_decode_step(q, k, v, kl, vl, out=out, alpha_out=alpha, ws=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    gen = torch.Generator(device=DEV).manual_seed(91)
    for r in range(4):
        print("case graph replay %d" % r, flush=True)
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
        k[:, :, : 64 * (r + 1)] = torch.randn((B, Hkv, 64 * (r + 1), 128), generator=gen, device=DEV).to(k.dtype)
        # an eager call of another shape on the same workspace, then the replay
        ops.cached_attn_lse(q[:, :8], k[:, :2, :3000].contiguous(), v[:, :2, :3000].contiguous(), ws=ws)
        g.replay()
        ops.dense_decode_step(q, k, v, kl, vl, out=ref_o, alpha_out=ref_a, ws=ws_ref)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(alpha, ref_a), "replay %d differs from the eager call" % r


def test_graph_replays_match_eager_shared_document(orc):
    """The shared-document decode step (64-row pass with local tokens, then the combine), captured once and
    replayed with new inputs and eager calls of other shapes on the same workspace in between: every
    replay equals an eager call bit for bit, and the last one matches the oracle."""
    B, Hq, Hkv, n, nl = 16, 32, 8, 5003, 300
    g0 = torch.Generator().manual_seed(95)
    q = torch.randn((B, Hq, 128), generator=g0).to(torch.bfloat16).to(DEV)
    k = torch.randn((1, Hkv, n, 128), generator=g0).to(torch.bfloat16).to(DEV)
    v = torch.randn((1, Hkv, n, 128), generator=g0).to(torch.bfloat16).to(DEV)
    kl = torch.randn((B, Hkv, nl, 128), generator=g0).to(torch.bfloat16).to(DEV)
    vl = torch.randn((B, Hkv, nl, 128), generator=g0).to(torch.bfloat16).to(DEV)
    n_loc = torch.tensor([(37 * i) % (nl + 1) for i in range(B)], dtype=torch.int32, device=DEV)
    nb = ops.ws_bytes_dense_decode_step(B, Hq, Hkv, 128, n, 0, nl)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    ws_ref = torch.empty(nb, dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, 128), device=DEV)
    alpha = torch.empty((B, Hq), device=DEV)
    ref_o = torch.empty_like(out)
    ref_a = torch.empty_like(alpha)

    def step():
        ops.dense_decode_step(q, k, v, kl, vl, n_loc, out=out, alpha_out=alpha, ws=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    gen = torch.Generator(device=DEV).manual_seed(96)
    for r in range(4):
        print("case shared-document graph replay %d" % r, flush=True)
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
        kl[:, :, : 32 * (r + 1)] = torch.randn((B, Hkv, 32 * (r + 1), 128), generator=gen, device=DEV).to(kl.dtype)
        k[:, :, : 64 * (r + 1)] = torch.randn((1, Hkv, 64 * (r + 1), 128), generator=gen, device=DEV).to(k.dtype)
        ops.cached_attn_lse(q[:4, :8].contiguous(), k[:, :2, :3000].contiguous(), v[:, :2, :3000].contiguous(), ws=ws)
        g.replay()
        ops.dense_decode_step(q, k, v, kl, vl, n_loc, out=ref_o, alpha_out=ref_a, ws=ws_ref)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(alpha, ref_a), "replay %d differs from the eager call" % r
    ro, ra = orc.dense_attn(to_np(q), to_np(k), to_np(v))
    mo, ma = orc.merge_local(to_np(q), ro, ra, to_np(kl), to_np(vl), to_np(n_loc))
    assert_close(out, alpha, mo, ma, torch.bfloat16, "shared-document replay vs oracle")
