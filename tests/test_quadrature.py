"""The Nectar quadrature module's evaluation, softmax(W q / sqrt d)^T Z and alpha = log sum exp(W q / sqrt d)
("Nectar: Neural Estimation of Cached-Token Attention via Regression", slide "The representation and the
loss are separate choices", quadrature block): cached_attn_lse with K = W and V = Z shared by every query,
at many query rows per KV head (the 64-row MFMA pass with several row groups).  Against the oracle's dense
attention; W and Z are random (their trained values are out of reach)."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import ops, synth
from tests.util import assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
CFG = synth.QUADRATURE


@pytest.mark.parametrize("B,p", [(64, 1000), (37, 6144), (8, 31)])
def test_quadrature_reduced(orc, B, p):
    """Every output row against the oracle: several 64-row groups (and a ragged one), p not a multiple of
    the 32-token block, and a module shorter than one block."""
    print("case quadrature B=%d p=%d" % (B, p), flush=True)
    x = synth.make_inputs(CFG, device=DEV, n=p, B=B)
    out, alpha = ops.cached_attn_lse(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    ro, ra = orc.dense_attn(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]))
    assert_close(out, alpha, ro, ra, torch.bfloat16, "quadrature B=%d p=%d" % (B, p))


def test_quadrature_full_size(orc):
    """The full shape (256 queries, p = 6,144): sampled queries, all their heads."""
    print("case quadrature full size B=%d p=%d" % (CFG.B, CFG.n), flush=True)
    x = synth.make_inputs(CFG, device=DEV)
    out, alpha = ops.cached_attn_lse(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    k, v = to_np(x["k"]), to_np(x["v"])
    for b in (0, 77, 128, 255):
        ro, ra = orc.dense_attn(to_np(x["q"][b:b + 1]), k, v)
        assert_close(out[b:b + 1], alpha[b:b + 1], ro, ra, torch.bfloat16, "quadrature query %d" % b)
