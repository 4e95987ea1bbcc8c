"""dense_decode_step_noalloc (the library's static scratch array instead of a caller workspace) against
dense_decode_step on the same inputs, through the C ABI: results must be identical, since both run the same
kernels in the same launch shapes; the oracle checks both to the usual bar.  Two calls in a row on each path,
the second with a smaller input, so the second call runs on whatever the first left in the array."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import ops
from tests.util import assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(B, Hq, Hkv, n, n_loc, dtype, seed, shared=False):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, 128), generator=g).to(dtype)
    Bk = 1 if shared else B
    k = torch.randn((Bk, Hkv, n, 128), generator=g).to(dtype)
    v = torch.randn((Bk, Hkv, n, 128), generator=g).to(dtype)
    nmax = max(n_loc)
    kl = torch.randn((B, Hkv, nmax, 128), generator=g).to(dtype)
    vl = torch.randn((B, Hkv, nmax, 128), generator=g).to(dtype)
    return q, k, v, kl, vl, torch.tensor(n_loc, dtype=torch.int32)


def _run(orc, B, Hq, Hkv, n, n_loc, dtype, seed, shared=False):
    print("case noalloc B=%d Hq=%d Hkv=%d n=%d n_loc=%s %s shared=%s" % (B, Hq, Hkv, n, n_loc, dtype, shared),
          flush=True)
    x = _case(B, Hq, Hkv, n, n_loc, dtype, seed, shared)
    q, k, v, kl, vl, nl = (t.to(DEV) for t in x)
    out = torch.full((B, Hq, 128), float("nan"), device=DEV)
    alpha = torch.full((B, Hq), float("nan"), device=DEV)
    ops.dense_decode_step_noalloc(q, k, v, kl, vl, nl, out=out, alpha_out=alpha)
    ref_o, ref_a = ops.dense_decode_step(q, k, v, kl, vl, nl)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o), "outputs differ from dense_decode_step"
    assert torch.equal(alpha, ref_a), "alphas differ from dense_decode_step"
    ro, ra = orc.dense_attn(to_np(x[0]), to_np(x[1]), to_np(x[2]))
    mo, ma = orc.merge_local(to_np(x[0]), ro, ra, to_np(x[3]), to_np(x[4]), x[5].numpy())
    assert_close(out, alpha, mo, ma, dtype, "noalloc step")


def test_noalloc_fused_one_cache_per_item(orc):
    """bf16, one cache per batch item: the single split launch whose last workgroup combines."""
    _run(orc, 2, 32, 8, 61440 // 4 + 5, [256, 100], torch.bfloat16, 9100)
    _run(orc, 1, 32, 8, 1000, [64], torch.bfloat16, 9101)


def test_noalloc_shared_document(orc):
    """A shared document read by more than 16 rows per KV head: the 64-row pass plus combine."""
    _run(orc, 16, 8, 2, 3000, [512] * 15 + [300], torch.bfloat16, 9200, shared=True)
    _run(orc, 8, 8, 2, 700, [64, 0, 33, 1, 64, 5, 31, 32], torch.bfloat16, 9201, shared=True)


def test_noalloc_two_call_form(orc):
    """fp32 (and a shared document read by few rows) run as cached_attn_lse then lse_merge_local."""
    _run(orc, 3, 8, 2, 900, [64, 3, 0], torch.float32, 9300)
    _run(orc, 2, 8, 2, 500, [32, 1], torch.bfloat16, 9301, shared=True)
