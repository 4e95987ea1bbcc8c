"""Dense path on the GPU (through the C ABI) against the CPU oracle, element by element.

cached_attn_lse: A and alpha; lse_merge_local: the exact merge with local tokens.
Bar: row-normwise relative error <= 2e-3 on outputs and <= 1e-3 absolute on alpha
for bf16 inputs; 1e-5 / 1e-5 for fp32 inputs (tests/util.py)."""
import numpy as np
import pytest
import torch

from long_context_decode_attn_amd import ops, synth
from tests.util import assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, Hq, Hkv, n, dtype, seed, shared=False, scale_q=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn((B, Hq, 128), generator=g) * scale_q).to(dtype)
    Bk = 1 if shared else B
    k = torch.randn((Bk, Hkv, n, 128), generator=g).to(dtype)
    v = torch.randn((Bk, Hkv, n, 128), generator=g).to(dtype)
    return q, k, v


def _dense_case(B, Hq, Hkv, n, dtype, seed, shared=False, scale_q=1.0, orc=None):
    q, k, v = _inputs(B, Hq, Hkv, n, dtype, seed, shared, scale_q)
    print("case dense B=%d Hq=%d Hkv=%d n=%d %s shared=%s" % (B, Hq, Hkv, n, dtype, shared), flush=True)
    out, alpha = ops.cached_attn_lse(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    ro, ra = orc.dense_attn(to_np(q), to_np(k), to_np(v))
    return assert_close(out, alpha, ro, ra, dtype, "dense B=%d Hq=%d Hkv=%d n=%d" % (B, Hq, Hkv, n))


@pytest.mark.parametrize("n", [1, 2, 31, 32, 33, 127, 128, 129, 1000, 4096, 5003])
def test_dense_bf16_lengths(orc, n):
    _dense_case(2, 8, 2, n, torch.bfloat16, 100 + n, orc=orc)


@pytest.mark.parametrize("n", [1, 17, 64, 1000, 4096])
def test_dense_fp32_lengths(orc, n):
    _dense_case(2, 8, 2, n, torch.float32, 200 + n, orc=orc)


@pytest.mark.parametrize("B,G", [(1, 1), (1, 2), (3, 3), (1, 8), (2, 16), (1, 32)])
def test_dense_gqa_shapes(orc, B, G):
    _dense_case(B, 2 * G, 2, 700, torch.bfloat16, 300 + B * G, orc=orc)
    _dense_case(B, 2 * G, 2, 300, torch.float32, 400 + B * G, orc=orc)


@pytest.mark.parametrize("B", [2, 4, 5, 8, 16, 20])
def test_dense_shared_document(orc, B):
    """One cached document read by B batch items: B*G rows share each KV head (MFMA tiles of 16/32/64 rows)."""
    _dense_case(B, 8, 2, 3000, torch.bfloat16, 500 + B, shared=True, orc=orc)


@pytest.mark.parametrize("B,n", [(5, 100), (8, 300), (16, 33), (16, 3000), (20, 5003), (32, 2048)])
def test_dense_shared_rows_kernel(orc, B, n):
    """More than 16 rows per KV head (B*G rows on one shared document): 64-row workgroups that read each block
    once into LDS; one split (rows finished in place, n <= 512) and several (in-kernel combine)."""
    _dense_case(B, 8, 2, n, torch.bfloat16, 700 + B + n, shared=True, orc=orc)


@pytest.mark.parametrize("variant", list(range(9)))
def test_dense_shared_rows_variants(orc, variant):
    """Every 64-row workgroup variant (LDS ring depths and occupancies, blocks in registers) gives the
    oracle's result, several blocks per workgroup and a ragged tail."""
    old = ops.get_tuning("rows_variant")
    ops.set_tuning("rows_variant", variant)
    try:
        _dense_case(16, 8, 2, 7680 + 5, torch.bfloat16, 780 + variant, shared=True, orc=orc)
        _dense_case(20, 8, 2, 3001, torch.bfloat16, 790 + variant, shared=True, orc=orc)
    finally:
        ops.set_tuning("rows_variant", old)


def test_dense_shared_rows_kernel_off(orc):
    """The same shapes through one-wavefront-per-32/64-rows tiles (rows_kernel = 0)."""
    old = ops.get_tuning("rows_kernel")
    ops.set_tuning("rows_kernel", 0)
    try:
        for B in (8, 16):
            _dense_case(B, 8, 2, 3000, torch.bfloat16, 760 + B, shared=True, orc=orc)
    finally:
        ops.set_tuning("rows_kernel", old)


def test_config3_reduced(orc):
    """Config 3 recipe (one shared document, 16 queries, 512 private local tokens each), one layer at
    n = 7,680: the decode step (document pass + local merge) against the oracle, every row."""
    cfg = synth.CONFIGS[3]
    x = synth.make_inputs(cfg, n=7680)
    print("case config 3 reduced", flush=True)
    out, alpha = ops.dense_decode_step(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), x["k_loc"].to(DEV),
                                       x["v_loc"].to(DEV), x["n_loc"].to(DEV))
    torch.cuda.synchronize()
    ro, ra = orc.dense_attn(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]))
    mo, ma = orc.merge_local(to_np(x["q"]), ro, ra, to_np(x["k_loc"]), to_np(x["v_loc"]), to_np(x["n_loc"]))
    assert_close(out, alpha, mo, ma, torch.bfloat16, "config 3 reduced step")


def test_config3_full_size_sampled(orc):
    """One layer of config 3 at full size (shared 61,440-token document, 16 queries x 32 heads, 512
    private local tokens each) through dense_decode_step, the call and launch shape the shared36
    benchmark times; every row of three batch items against the oracle."""
    cfg = synth.CONFIGS[3]
    x = synth.make_inputs(cfg, device=DEV)
    print("case config 3 full size n=%d B=%d" % (cfg.n, cfg.B), flush=True)
    out, alpha = ops.dense_decode_step(x["q"], x["k"], x["v"], x["k_loc"], x["v_loc"], x["n_loc"])
    torch.cuda.synchronize()
    k, v = to_np(x["k"]), to_np(x["v"])
    for b in (0, 7, 15):
        q = to_np(x["q"][b:b + 1])
        ro, ra = orc.dense_attn(q, k, v)
        mo, ma = orc.merge_local(q, ro, ra, to_np(x["k_loc"][b:b + 1]), to_np(x["v_loc"][b:b + 1]),
                                 to_np(x["n_loc"][b:b + 1]))
        assert_close(out[b:b + 1], alpha[b:b + 1], mo, ma, torch.bfloat16, "config 3 full size b=%d" % b)


def test_dense_fp32_shared_document(orc):
    _dense_case(3, 8, 2, 2000, torch.float32, 600, shared=True, orc=orc)


def test_dense_large_logits(orc):
    """Peaked softmax (|s| up to ~100): exercises the running-max rescale."""
    _dense_case(2, 8, 2, 3000, torch.bfloat16, 700, scale_q=8.0, orc=orc)
    _dense_case(1, 4, 1, 3000, torch.float32, 701, scale_q=8.0, orc=orc)


def test_dense_increasing_logits(orc):
    """Logits growing along the sequence force a rescale in almost every block."""
    B, Hq, Hkv, n = 1, 4, 1, 4000
    q = torch.zeros((B, Hq, 128))
    q[..., 0] = 1.0
    k = torch.randn((B, Hkv, n, 128)) * 0.1
    k[..., 0] = torch.linspace(0, 400, n)
    v = torch.randn((B, Hkv, n, 128))
    for dt in (torch.bfloat16, torch.float32):
        qq, kk, vv = q.to(dt), k.to(dt), v.to(dt)
        out, alpha = ops.cached_attn_lse(qq.to(DEV), kk.to(DEV), vv.to(DEV))
        ro, ra = orc.dense_attn(to_np(qq), to_np(kk), to_np(vv))
        assert_close(out, alpha, ro, ra, dt, "increasing logits %s" % dt)


def test_dense_empty_cache(orc):
    q, k, v = _inputs(2, 8, 2, 0, torch.bfloat16, 800)
    out, alpha = ops.cached_attn_lse(q.to(DEV), k.to(DEV), v.to(DEV))
    assert torch.all(out == 0) and torch.all(torch.isneginf(alpha))


def test_dense_config1_tiny_fp32(orc):
    cfg = synth.CONFIGS[1]
    x = synth.make_inputs(cfg)
    out, alpha = ops.cached_attn_lse(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV))
    ro, ra = orc.dense_attn(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]))
    assert_close(out, alpha, ro, ra, torch.float32, "config 1")
    mo, ma = ops.lse_merge_local(x["q"].to(DEV), out, alpha, x["k_loc"].to(DEV), x["v_loc"].to(DEV),
                                 x["n_loc"].to(DEV))
    rmo, rma = orc.merge_local(to_np(x["q"]), ro, ra, to_np(x["k_loc"]), to_np(x["v_loc"]), to_np(x["n_loc"]))
    assert_close(mo, ma, rmo, rma, torch.float32, "config 1 merge")


# ------------------------------------------------------------------ merge ----
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_merge_ragged_local(orc, dtype):
    B, Hq, Hkv, n, nl = 4, 8, 2, 900, 300
    q, k, v = _inputs(B, Hq, Hkv, n, dtype, 900)
    g = torch.Generator().manual_seed(901)
    kl = torch.randn((B, Hkv, nl, 128), generator=g).to(dtype)
    vl = torch.randn((B, Hkv, nl, 128), generator=g).to(dtype)
    n_loc = torch.tensor([0, 1, 37, 300], dtype=torch.int32)
    a, al = ops.cached_attn_lse(q.to(DEV), k.to(DEV), v.to(DEV))
    mo, ma = ops.lse_merge_local(q.to(DEV), a, al, kl.to(DEV), vl.to(DEV), n_loc.to(DEV))
    # kernel isolation: the oracle merges the GPU's own (A, alpha)
    ro, ra = orc.merge_local(to_np(q), a.cpu().numpy(), al.cpu().numpy(), to_np(kl), to_np(vl), n_loc.numpy())
    assert_close(mo, ma, ro, ra, dtype, "merge (GPU A, alpha)")
    # end to end against dense attention over the concatenation
    for b in range(B):
        kk = torch.cat([k[b:b + 1], kl[b:b + 1, :, :int(n_loc[b])]], dim=2)
        vv = torch.cat([v[b:b + 1], vl[b:b + 1, :, :int(n_loc[b])]], dim=2)
        fo, fa = orc.dense_attn(to_np(q[b:b + 1]), to_np(kk), to_np(vv))
        assert_close(mo[b:b + 1], ma[b:b + 1], fo, fa, dtype, "merge end-to-end b=%d" % b)


def test_merge_fed_oracle_state(orc):
    """lse_merge_local fed the oracle's (A, alpha), so a failure points at the merge alone."""
    B, Hq, Hkv, n, nl = 2, 8, 2, 500, 256
    q, k, v = _inputs(B, Hq, Hkv, n, torch.bfloat16, 950)
    g = torch.Generator().manual_seed(951)
    kl = torch.randn((B, Hkv, nl, 128), generator=g).to(torch.bfloat16)
    vl = torch.randn((B, Hkv, nl, 128), generator=g).to(torch.bfloat16)
    ro, ra = orc.dense_attn(to_np(q), to_np(k), to_np(v))
    a = torch.from_numpy(ro.astype(np.float32)).to(DEV)
    al = torch.from_numpy(ra.astype(np.float32)).to(DEV)
    mo, ma = ops.lse_merge_local(q.to(DEV), a, al, kl.to(DEV), vl.to(DEV))
    rmo, rma = orc.merge_local(to_np(q), ro.astype(np.float32), ra.astype(np.float32), to_np(kl), to_np(vl))
    assert_close(mo, ma, rmo, rma, torch.bfloat16, "merge fed oracle state")


def test_merge_empty_sides(orc):
    B, Hq, Hkv, nl = 2, 8, 2, 64
    q, kl, vl = _inputs(B, Hq, Hkv, nl, torch.bfloat16, 960)
    a = torch.zeros((B, Hq, 128), device=DEV)
    al = torch.full((B, Hq), float("-inf"), device=DEV)
    mo, ma = ops.lse_merge_local(q.to(DEV), a, al, kl.to(DEV), vl.to(DEV))
    ro, ra = orc.dense_attn(to_np(q), to_np(kl), to_np(vl))
    assert_close(mo, ma, ro, ra, torch.bfloat16, "merge with empty cached part")
    mo, ma = ops.lse_merge_local(q.to(DEV), a, al, kl.to(DEV), vl.to(DEV),
                                 torch.zeros(B, dtype=torch.int32, device=DEV))
    assert torch.all(mo == 0) and torch.all(torch.isneginf(ma))


# ------------------------------------------------------------- full sizes ----
def test_config2_full_size(orc):
    """Qwen3-4B-shaped layer at full size: n = 61,440, 8 KV heads, 32 query heads, 256 local tokens;
    every output row checked."""
    cfg = synth.CONFIGS[2]
    x = synth.make_inputs(cfg)
    print("case config 2 full size", flush=True)
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    a, al = ops.cached_attn_lse(q, k, v)
    mo, ma = ops.lse_merge_local(q, a, al, x["k_loc"].to(DEV), x["v_loc"].to(DEV), x["n_loc"].to(DEV))
    torch.cuda.synchronize()
    ro, ra = orc.dense_attn(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]))
    assert_close(a, al, ro, ra, torch.bfloat16, "config 2 cached part")
    rmo, rma = orc.merge_local(to_np(x["q"]), ro, ra, to_np(x["k_loc"]), to_np(x["v_loc"]), to_np(x["n_loc"]))
    assert_close(mo, ma, rmo, rma, torch.bfloat16, "config 2 merged")


# ------------------------------------------------------ fused decode step ----
def _step_case(orc, B, Hq, Hkv, n, nl_max, n_loc, dtype, seed, shared=False, doc=False):
    q, k, v = _inputs(B, Hq, Hkv, n, dtype, seed, shared)
    g = torch.Generator().manual_seed(seed + 1)
    kl = torch.randn((B, Hkv, nl_max, 128), generator=g).to(dtype)
    vl = torch.randn((B, Hkv, nl_max, 128), generator=g).to(dtype)
    nlt = torch.tensor(n_loc, dtype=torch.int32)
    print("case step B=%d Hq=%d Hkv=%d n=%d n_loc=%s %s shared=%s doc=%s" % (B, Hq, Hkv, n, n_loc, dtype, shared, doc),
          flush=True)
    a_doc = torch.empty((B, Hq, 128), device=DEV) if doc else None
    al_doc = torch.empty((B, Hq), device=DEV) if doc else None
    out, alpha = ops.dense_decode_step(q.to(DEV), k.to(DEV), v.to(DEV), kl.to(DEV), vl.to(DEV), nlt.to(DEV),
                                       a_doc=a_doc, alpha_doc=al_doc)
    torch.cuda.synchronize()
    ro, ra = orc.dense_attn(to_np(q), to_np(k), to_np(v))
    mo, ma = orc.merge_local(to_np(q), ro, ra, to_np(kl), to_np(vl), nlt.numpy())
    assert_close(out, alpha, mo, ma, dtype, "decode step")
    if doc:
        assert_close(a_doc, al_doc, ro, ra, dtype, "decode step doc-only part")


@pytest.mark.parametrize("n,n_loc", [(61440 // 16, [256]), (1000, [0, 17, 256]), (31, [5, 40]), (4096, [300, 0]),
                                     (1, [1, 64]), (5003, [64, 64])])
def test_decode_step_fused(orc, n, n_loc):
    """Cache and local tokens as one token range (cache length not a multiple of 32: the local tokens start at
    the next block boundary and the gap is masked)."""
    _step_case(orc, len(n_loc), 32, 8, n, max(n_loc), n_loc, torch.bfloat16, 1000 + n)


@pytest.mark.parametrize("B,Hq,n,n_loc", [
    (16, 8, 3000, [512] * 15 + [300]),                      # 64 rows: one 64-row group, one local block per wavefront
    (20, 8, 5003, [(37 * i) % 301 for i in range(20)]),     # 80 rows: two groups, ragged and empty local ranges
    (11, 6, 2000, [(53 * i) % 130 + 1 for i in range(11)]),  # G = 3: a wavefront's rows span parts of items
    (16, 8, 200, [700] * 16),                               # few splits: several local blocks per wavefront
    (8, 8, 20, [64, 0, 33, 1, 64, 5, 31, 32]),              # one block: one split, rows finished in place
])
def test_decode_step_shared_rows_local(orc, B, Hq, n, n_loc):
    """A shared document with more than 16 rows per KV head: the 64-row pass also takes each row's local
    tokens (blocks seen only by that item's rows), then one combine."""
    _step_case(orc, B, Hq, 2, n, max(n_loc), n_loc, torch.bfloat16, 1200 + B + n, shared=True)


@pytest.mark.parametrize("variant", [0, 7, 8])
def test_decode_step_shared_rows_local_variants(orc, variant):
    """The shared-document step with local tokens through each ring variant that takes them: 64 and 80 rows,
    ragged and empty local ranges, G = 3, several local blocks per wavefront, one split finished in place."""
    old = ops.get_tuning("rows_variant")
    ops.set_tuning("rows_variant", variant)
    try:
        _step_case(orc, 16, 8, 2, 3000, 512, [512] * 15 + [300], torch.bfloat16, 1300 + variant, shared=True)
        _step_case(orc, 20, 8, 2, 5003, 300, [(37 * i) % 301 for i in range(20)], torch.bfloat16, 1310 + variant,
                   shared=True)
        _step_case(orc, 11, 6, 2, 2000, 130, [(53 * i) % 130 + 1 for i in range(11)], torch.bfloat16,
                   1320 + variant, shared=True)
        _step_case(orc, 16, 8, 2, 200, 700, [700] * 16, torch.bfloat16, 1330 + variant, shared=True)
        _step_case(orc, 8, 8, 2, 20, 64, [64, 0, 33, 1, 64, 5, 31, 32], torch.bfloat16, 1340 + variant, shared=True)
        _step_case(orc, 16, 8, 2, 61440 // 8 + 7, 512, [512] * 16, torch.bfloat16, 1350 + variant, shared=True)
    finally:
        ops.set_tuning("rows_variant", old)


def test_decode_step_fallbacks(orc):
    """fp32, a shared document, and doc-only outputs run as the two separate calls."""
    _step_case(orc, 2, 8, 2, 700, 64, [64, 3], torch.float32, 1100)
    _step_case(orc, 3, 8, 2, 900, 32, [32, 1, 0], torch.bfloat16, 1101, shared=True)
    _step_case(orc, 2, 8, 2, 800, 48, [48, 10], torch.bfloat16, 1102, doc=True)
    _step_case(orc, 2, 8, 2, 0, 48, [48, 10], torch.bfloat16, 1103)


def test_decode_step_config2_full_size(orc):
    cfg = synth.CONFIGS[2]
    x = synth.make_inputs(cfg)
    out, alpha = ops.dense_decode_step(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), x["k_loc"].to(DEV),
                                       x["v_loc"].to(DEV), x["n_loc"].to(DEV))
    torch.cuda.synchronize()
    ro, ra = orc.dense_attn(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]))
    mo, ma = orc.merge_local(to_np(x["q"]), ro, ra, to_np(x["k_loc"]), to_np(x["v_loc"]), to_np(x["n_loc"]))
    assert_close(out, alpha, mo, ma, torch.bfloat16, "config 2 fused step")


# ------------------------------------------------------- kernel variants ----
@pytest.mark.parametrize("variant,wgs", [(0, 256), (1, 256), (2, 256), (3, 256), (3, 512), (3, 1024), (4, 256)])
def test_dense_split_variants(orc, variant, wgs):
    """Every MFMA split variant (nontemporal / cached loads, one or two blocks ahead, two waves per SIMD), the bf16
    VALU split kept for comparison (variant 4), and launch width give the oracle's result, for the plain call and
    the fused step, ragged and short ranges."""
    old = ops.get_tuning("dense_variant")
    old_w = ops.get_tuning("dense_wgs")
    ops.set_tuning("dense_variant", variant)
    ops.set_tuning("dense_wgs", wgs)
    try:
        for n in (33, 1000, 5003, 61440 // 8):
            _dense_case(2, 8, 2, n, torch.bfloat16, 1200 + n + variant, orc=orc)
        _step_case(orc, 2, 32, 8, 3001, 200, [200, 7], torch.bfloat16, 1300 + variant)
        _step_case(orc, 1, 32, 8, 4096, 256, [256], torch.bfloat16, 1310 + variant)
    finally:
        ops.set_tuning("dense_variant", old)
        ops.set_tuning("dense_wgs", old_w)


# -------------------------------------------------------- combine slots ----
@pytest.mark.parametrize("wgs,n", [(2, 20800), (4, 20800), (5, 20800), (8, 20800), (9, 20800), (16, 20800),
                                   (17, 20800), (32, 20800), (33, 20800), (64, 20480), (65, 20800), (200, 20800)])
def test_combine_slot_counts(orc, wgs, n):
    """fp32 split over one KV head with valu_wgs target workgroups: 2, 4, 5, 8, 9, 16, 17, 32, 33, 64, 65 and 186
    slots per row (16-token blocks, 1,300 or 1,280 of them), on both sides of each slot bound of the
    one-wavefront-per-row combine and of the switch to a workgroup per row past 64 slots; cached_attn_lse, and the
    fused step whose merge with local tokens enters as the virtual pair."""
    old = ops.get_tuning("valu_wgs")
    ops.set_tuning("valu_wgs", wgs)
    try:
        _dense_case(1, 4, 1, n, torch.float32, 1500 + wgs, orc=orc)
        _step_case(orc, 1, 4, 1, n, 100, [100], torch.float32, 1600 + wgs)
    finally:
        ops.set_tuning("valu_wgs", old)
