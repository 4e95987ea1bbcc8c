"""Seeded synthetic inputs for decode attention against a cached K/V.

This module only draws inputs.  It holds none of the attention, scoring or
selection arithmetic: signatures are produced here as *inputs* (sign bits of
a seeded random projection, the random-projection stand-in for a learned
signature map), and both the GPU library and the CPU oracle receive the same
arrays.

Recipe
------
* Every tensor slice has its own ``torch.Generator`` seeded with
  ``seed(config, slot, rot, b, h)``:
  ``1_000_000 * b_h + 1000 * config + 100 * rot + slot`` where ``b_h`` numbers
  the (batch, head) slice (0 when the tensor is drawn whole).  The slot
  numbers are fixed below.
* Values are fp32 N(0, 1) draws, rounded to bf16 with round-to-nearest-even
  (``Tensor.to(torch.bfloat16)``) when the dtype is bf16.
* The generator lives on the device the tensor is made on; a CPU draw and a
  GPU draw with the same seed give different (equally distributed) numbers.
  Parity tests draw on the CPU and upload; the benchmark draws on the GPU.
* Key/query signatures: bit j (LSB = 0) of the 32-bit code of x is
  ``[(x @ R)_j > 0]`` with one shared projection ``R`` in R^{d x 32}, iid
  N(0, 1), drawn in float64 and applied in float64 to the (bf16-rounded)
  vectors.
* Needles: for each (b, KV head h), 64 distinct positions uniform in
  [128, n - 128); each key there is replaced by bf16(4 * q[b, G*h] + eps),
  eps ~ N(0, I) (``4x the query direction`` read literally as 4 * q).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

SLOT = {"q": 0, "k": 1, "v": 2, "k_loc": 3, "v_loc": 4, "proj": 5, "needles": 6,
        "key_sigs": 7, "q_sigs": 8, "n_loc": 9}


def seed(config: int, slot: str, rot: int = 0, bh: int = 0) -> int:
    return 1_000_000 * bh + 1000 * config + 100 * rot + SLOT[slot]


def _gen(s: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(s))
    return g


def normal(shape, s: int, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """fp32 N(0,1) draws from one generator seeded with ``s``, cast to ``dtype``."""
    x = torch.randn(tuple(shape), generator=_gen(s, device), device=device, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def normal_sliced(lead, tail, config: int, slot: str, rot: int = 0, dtype=torch.bfloat16,
                  device="cpu") -> torch.Tensor:
    """Tensor of shape lead + tail whose every leading slice has its own seed.

    Drawing slice by slice keeps the fp32 staging buffer at one slice and lets
    a checker regenerate any single slice on its own."""
    lead = tuple(lead)
    out = torch.empty(lead + tuple(tail), dtype=dtype, device=device)
    flat = out.view(-1, *tail)
    for i in range(flat.shape[0]):
        flat[i] = normal(tail, seed(config, slot, rot, i), dtype, device)
    return out


def projection(d: int, bits: int, config: int, device="cpu") -> torch.Tensor:
    """R in R^{d x bits}, iid N(0,1), float64."""
    g = _gen(seed(config, "proj"), device)
    return torch.randn((d, bits), generator=g, device=device, dtype=torch.float64)


def signatures(x: torch.Tensor, R: torch.Tensor, chunk: int = 1 << 20) -> torch.Tensor:
    """Pack the sign bits of x @ R (last dim of x = d) into uint32 codes (as int32 storage)."""
    lead = x.shape[:-1]
    xf = x.reshape(-1, x.shape[-1])
    bits = R.shape[1]
    assert bits == 32
    weights = (torch.ones(bits, dtype=torch.int64, device=x.device) << torch.arange(bits, device=x.device))
    out = torch.empty(xf.shape[0], dtype=torch.int64, device=x.device)
    for s in range(0, xf.shape[0], chunk):
        p = xf[s:s + chunk].to(torch.float64) @ R.to(x.device)
        out[s:s + chunk] = ((p > 0).to(torch.int64) * weights).sum(-1)
    # values in [0, 2^32); keep the bit pattern in int32 storage (uint32 semantics)
    out = torch.where(out >= (1 << 31), out - (1 << 32), out).to(torch.int32)
    return out.view(lead)


def as_uint32_numpy(sig: torch.Tensor):
    return sig.cpu().numpy().view("uint32")


def plant_needles(k: torch.Tensor, q: torch.Tensor, config: int, count: int = 64, margin: int = 128):
    """In place: k [B, Hkv, n, d], q [B, Hq, d].  Returns positions [B, Hkv, count] (int64, sorted)."""
    B, Hkv, n, d = k.shape
    G = q.shape[1] // Hkv
    dev = k.device
    pos_all = torch.empty((B, Hkv, count), dtype=torch.int64, device=dev)
    for b in range(B):
        for h in range(Hkv):
            g = _gen(seed(config, "needles", 0, b * Hkv + h), dev)
            perm = torch.randperm(n - 2 * margin, generator=g, device=dev)[:count] + margin
            pos = torch.sort(perm).values
            eps = torch.randn((count, d), generator=g, device=dev, dtype=torch.float32)
            direction = q[b, G * h].to(torch.float32)
            k[b, h, pos] = (4.0 * direction[None, :] + eps).to(k.dtype)
            pos_all[b, h] = pos
    return pos_all


@dataclass
class Config:
    """One workload: the shapes and knobs of a decode step."""
    cid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    n: int
    dtype: torch.dtype
    n_loc: int = 0               # local tokens merged after the cached part
    shared_doc: bool = False     # one cached document read by every batch item
    layers: int = 1
    m: int = 0                   # retrieval budget (0: no sparse step)
    n_sink: int = 0
    n_recent: int = 0
    needles: int = 0
    sig_kind: str = "projection"  # "projection" (sign bits of x @ R) or "uniform" (random codes)
    extra: dict = field(default_factory=dict)


CONFIGS = {
    1: Config(1, "tiny fp32: Hkv=1 Hq=4 d=128 n=4096, 64 local, m=128+16 sink+64 recent",
              B=1, Hq=4, Hkv=1, d=128, n=4096, dtype=torch.float32, n_loc=64,
              m=128, n_sink=16, n_recent=64, sig_kind="uniform"),
    2: Config(2, "Qwen3-4B-shaped layer: Hkv=8 Hq=32 d=128 n=61440 bf16, B=1, 256 local",
              B=1, Hq=32, Hkv=8, d=128, n=61440, dtype=torch.bfloat16, n_loc=256),
    3: Config(3, "Qwen3-4B-shaped 36-layer shared document: Hkv=8 Hq=32 d=128 n=61440 bf16, "
                 "16 queries, 512 private local each",
              B=16, Hq=32, Hkv=8, d=128, n=61440, dtype=torch.bfloat16, n_loc=512,
              shared_doc=True, layers=36),
    4: Config(4, "HashAttention sparse: Hkv=8 Hq=32 d=128 n=131072 bf16, B=8, m=n/32+128+128",
              B=8, Hq=32, Hkv=8, d=128, n=131072, dtype=torch.bfloat16,
              m=131072 // 32, n_sink=128, n_recent=128),
    5: Config(5, "planted needles: Hkv=8 Hq=32 d=128 n=524288 bf16, B=4, dense vs sparse m=n/64",
              B=4, Hq=32, Hkv=8, d=128, n=524288, dtype=torch.bfloat16,
              m=524288 // 64, n_sink=128, n_recent=128, needles=64),
}

# A workload the same kernels serve beyond the five above: the Nectar quadrature
# module's evaluation, softmax(W q / sqrt d)^T Z with alpha = log sum exp(W q /
# sqrt d) ("Nectar: Neural Estimation of Cached-Token Attention via Regression",
# slide "The representation and the loss are separate choices", quadrature
# block), which is cached_attn_lse with K = W and V = Z.  p = 6,144 pairs per (layer, KV head) is the 10 % module of
# the 61,440-token document (Table 9's 914 MB over 36 layers x 8 KV heads x 512
# B per pair); 256 decode queries share it, so each KV head has 1,024 query rows
# and the contraction is dense.  W and Z are random (their quality needs trained
# values).
QUADRATURE = Config(6, "Nectar quadrature module: Hkv=8 Hq=32 d=128 p=6144 pairs (10% of 61,440) bf16, "
                       "256 queries sharing it",
                    B=256, Hq=32, Hkv=8, d=128, n=6144, dtype=torch.bfloat16, shared_doc=True)


def make_inputs(cfg: Config, device="cpu", rot: int = 0, n: int | None = None, B: int | None = None,
                layer: int = 0, with_sigs: bool | None = None, n_loc=None):
    """Draw one input set for ``cfg`` (optionally shrunk to n tokens / B queries).

    Returns a dict of tensors on ``device``:
      q [B,Hq,d]; k, v [Bkv,Hkv,n,d] (Bkv = 1 for a shared document);
      k_loc, v_loc [B,Hkv,n_loc_max,d] and n_loc [B] int32 when cfg.n_loc;
      key_sigs [Bkv,Hkv,n], q_sigs [B,Hq] (int32 storage of uint32 codes) when sparse;
      needle_pos [B,Hkv,count] when cfg.needles.
    ``layer`` shifts the seeds so each layer of a stack has its own tensors."""
    n = cfg.n if n is None else n
    B = cfg.B if B is None else B
    c = cfg.cid + 10 * layer
    Bkv = 1 if cfg.shared_doc else B
    out = {}
    out["q"] = normal_sliced((B,), (cfg.Hq, cfg.d), c, "q", rot, cfg.dtype, device)
    out["k"] = normal_sliced((Bkv, cfg.Hkv), (n, cfg.d), c, "k", rot, cfg.dtype, device)
    out["v"] = normal_sliced((Bkv, cfg.Hkv), (n, cfg.d), c, "v", rot, cfg.dtype, device)
    if cfg.n_loc:
        nl = cfg.n_loc if n_loc is None else n_loc
        if isinstance(nl, int):
            nmax = nl
            nl_t = torch.full((B,), nl, dtype=torch.int32)
        else:
            nl_t = torch.as_tensor(nl, dtype=torch.int32)
            nmax = int(nl_t.max().item()) if nl_t.numel() else 0
        out["k_loc"] = normal_sliced((B, cfg.Hkv), (nmax, cfg.d), c, "k_loc", rot, cfg.dtype, device)
        out["v_loc"] = normal_sliced((B, cfg.Hkv), (nmax, cfg.d), c, "v_loc", rot, cfg.dtype, device)
        out["n_loc"] = nl_t.to(device)
    if cfg.needles:
        out["needle_pos"] = plant_needles(out["k"], out["q"], c, cfg.needles)
    if with_sigs is None:
        with_sigs = cfg.m > 0
    if with_sigs and cfg.sig_kind == "uniform":
        out["key_sigs"] = uniform_sigs((Bkv, cfg.Hkv, n), seed(c, "key_sigs", rot), device)
        out["q_sigs"] = uniform_sigs((B, cfg.Hq), seed(c, "q_sigs", rot), device)
    elif with_sigs:
        R = projection(cfg.d, 32, c, device)
        out["key_sigs"] = signatures(out["k"], R)
        out["q_sigs"] = signatures(out["q"], R)
    return out


def uniform_sigs(shape, s: int, device="cpu") -> torch.Tensor:
    """Uniformly random 32-bit codes (int32 storage)."""
    g = _gen(s, device)
    return torch.randint(-(1 << 31), 1 << 31, tuple(shape), generator=g, device=device, dtype=torch.int64).to(torch.int32)
