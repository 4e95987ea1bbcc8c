"""The Python binding checks every tensor before a launch: host tensors, wrong shapes, dtypes, devices and short
workspaces raise ValueError, so that no host pointer or short buffer ever reaches a kernel.  The host-tensor cases
run without a GPU (the check comes before any library call that touches the device); the shape cases need GPU
tensors and run on the GPU, where they still raise before any launch."""
import os

import pytest
import torch

from long_context_decode_attn_amd import ops


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(ops.LIB_PATH):
        pytest.skip("liblcda.so not built")
    return ops.load()


def host_inputs(B=1, Hq=4, Hkv=1, n=64, cap=16, dtype=torch.bfloat16):
    return dict(q=torch.zeros(B, Hq, 128, dtype=dtype), k=torch.zeros(B, Hkv, n, 128, dtype=dtype),
                v=torch.zeros(B, Hkv, n, 128, dtype=dtype), k_loc=torch.zeros(B, Hkv, 8, 128, dtype=dtype),
                v_loc=torch.zeros(B, Hkv, 8, 128, dtype=dtype), key_sigs=torch.zeros(B, Hkv, n, dtype=torch.int32),
                q_sigs=torch.zeros(B, Hq, dtype=torch.int32), idx=torch.zeros(B, Hq, cap, dtype=torch.int32),
                count=torch.zeros(B, Hq, dtype=torch.int32), R=torch.zeros(128, 32))


CALLS = {
    "cached_attn_lse": lambda x: ops.cached_attn_lse(x["q"], x["k"], x["v"]),
    "lse_merge_local": lambda x: ops.lse_merge_local(x["q"], torch.zeros(1, 4, 128), torch.zeros(1, 4), x["k_loc"],
                                                     x["v_loc"]),
    "dense_decode_step": lambda x: ops.dense_decode_step(x["q"], x["k"], x["v"], x["k_loc"], x["v_loc"]),
    "dense_decode_step_noalloc": lambda x: ops.dense_decode_step_noalloc(x["q"], x["k"], x["v"], x["k_loc"],
                                                                         x["v_loc"]),
    "sig_score_topk": lambda x: ops.sig_score_topk(x["key_sigs"], x["q_sigs"], 8, 2, 2),
    "sig_score_topk_q": lambda x: ops.sig_score_topk_q(x["key_sigs"], x["q"], x["R"], 8, 2, 2),
    "sig_score_topk_w": lambda x: ops.sig_score_topk_w(x["key_sigs"].unsqueeze(-1).contiguous(),
                                                       x["q_sigs"].unsqueeze(-1).contiguous(), 8, 2, 2),
    "sig_encode": lambda x: ops.sig_encode(x["q"], x["R"]),
    "gather_attn": lambda x: ops.gather_attn(x["q"], x["k"], x["v"], x["idx"], x["count"]),
    "sparse_decode_step": lambda x: ops.sparse_decode_step(x["key_sigs"], x["q_sigs"], x["q"], x["k"], x["v"], 8, 2,
                                                           2),
}


@pytest.mark.parametrize("name", sorted(CALLS))
def test_host_tensors_are_refused(name):
    with pytest.raises(ValueError, match="GPU|must be on"):
        CALLS[name](host_inputs())


def gpu_inputs(**kw):
    return {k: v.cuda() for k, v in host_inputs(**kw).items()}


@pytest.mark.gpu
def test_gpu_shape_and_dtype_mismatches_raise_before_launch():
    x = gpu_inputs()
    dev = x["q"].device
    cases = [
        # caller-provided outputs of the wrong shape, dtype or device
        (lambda: ops.cached_attn_lse(x["q"], x["k"], x["v"], out=torch.empty(1, 4, 64, device=dev)), "out"),
        (lambda: ops.cached_attn_lse(x["q"], x["k"], x["v"], alpha=torch.empty(1, 4, dtype=torch.float64,
                                                                               device=dev)), "alpha"),
        (lambda: ops.cached_attn_lse(x["q"], x["k"], x["v"], out=torch.empty(1, 4, 128)), "out"),
        (lambda: ops.cached_attn_lse(x["q"], x["k"].cpu(), x["v"]), "K"),
        (lambda: ops.cached_attn_lse(x["q"], x["k"], x["v"], ws=torch.empty(16, dtype=torch.uint8, device=dev)),
         "workspace"),
        (lambda: ops.cached_attn_lse(x["q"], x["k"], x["v"], ws=torch.empty(1 << 20, dtype=torch.uint8)), "ws"),
        (lambda: ops.cached_attn_lse(x["q"], x["k"].float(), x["v"]), "dtype"),
        (lambda: ops.lse_merge_local(x["q"], torch.zeros(1, 4, 64, device=dev), torch.zeros(1, 4, device=dev),
                                     x["k_loc"], x["v_loc"]), "a_in"),
        (lambda: ops.lse_merge_local(x["q"], torch.zeros(1, 4, 128, device=dev), torch.zeros(1, 4, device=dev),
                                     x["k_loc"], x["v_loc"], n_loc=torch.zeros(1, dtype=torch.int64, device=dev)),
         "n_loc"),
        (lambda: ops.dense_decode_step(x["q"], x["k"], x["v"], x["k_loc"], x["v_loc"],
                                       a_doc=torch.zeros(1, 4, 128, device=dev)), "alpha_doc"),
        # index lists: idx of a smaller capacity than the call needs, or the wrong batch / head shape
        (lambda: ops.sig_score_topk(x["key_sigs"], x["q_sigs"], 8, 2, 2,
                                    idx=torch.zeros(1, 4, 4, dtype=torch.int32, device=dev)), "idx"),
        (lambda: ops.sig_score_topk(x["key_sigs"], x["q_sigs"][:, :2].contiguous().expand(2, 2).contiguous(), 8, 2,
                                    2), "q_sigs"),
        (lambda: ops.sig_score_topk(x["key_sigs"], x["q_sigs"], 8, 2, 2,
                                    count=torch.zeros(1, 4, dtype=torch.int64, device=dev)), "count"),
        (lambda: ops.sig_score_topk(x["key_sigs"].cpu(), x["q_sigs"], 8, 2, 2), "GPU"),
        (lambda: ops.sig_score_topk_q(x["key_sigs"], x["q"], x["R"], 8, 2, 2,
                                      q_sigs=torch.zeros(1, 3, dtype=torch.int32, device=dev)), "q_sigs"),
        (lambda: ops.gather_attn(x["q"], x["k"], x["v"], x["idx"][:, :2].contiguous(), x["count"]), "idx"),
        (lambda: ops.gather_attn(x["q"], x["k"], x["v"], x["idx"], x["count"][:, :2].contiguous()), "count"),
        (lambda: ops.gather_attn(x["q"], x["k"], x["v"], x["idx"].cpu(), x["count"]), "idx"),
        (lambda: ops.gather_attn(x["q"], x["k"], x["v"], x["idx"], x["count"].cpu()), "count"),
        (lambda: ops.sparse_decode_step(x["key_sigs"][:, :, :32].contiguous(), x["q_sigs"], x["q"], x["k"], x["v"],
                                        8, 2, 2), "key_sigs"),
        (lambda: ops.sparse_decode_step(x["key_sigs"], x["q_sigs"], x["q"], x["k"], x["v"], 8, 2, 2,
                                        idx=torch.zeros(1, 4, 5, dtype=torch.int32, device=dev)), "idx"),
        (lambda: ops.sig_encode(x["q"], x["R"], codes=torch.zeros(1, 4, dtype=torch.int32)), "codes"),
    ]
    for fn, text in cases:
        with pytest.raises(ValueError, match=text):
            fn()
    torch.cuda.synchronize()   # nothing was launched, nothing faulted
