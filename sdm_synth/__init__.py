"""Seeded synthetic inputs for the SDM hot path.

This module only draws numbers: it holds none of the method's arithmetic
(no scores, no selection, no update).  Both the CPU oracle and the HIP path
consume what it produces, so it is the single place where inputs come from.

Distributions follow the workload description of the Sparse Delta Memory
layer (queries/keys/values standard normal, sub-keys with variance
1/(d_k/2), forget gate a = sigmoid(N(3,1)), input gate b = sigmoid(N(0,1)),
learned initial memory M0 with variance 0.02).  The second parameter of
N(mean, x) is read as a variance.

Two backends:
  * ``numpy``  - PCG64 on the host, one spawned sub-stream per tensor in the
    fixed order C, k, q, v, a, b, M0, masks.  Used for every size the CPU
    oracle handles in full.
  * ``torch``  - a seeded torch generator on the GPU for the large layers whose
    inputs are too big to draw on the host quickly; tests copy the sampled
    slices back to the host for the oracle.
bf16 inputs are produced once by round-to-nearest-even from fp32 draws and
are the ground truth for both sides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = ["Dims", "PRESETS", "preset", "make_inputs", "make_layer_edge_inputs", "make_layer_edge_grads", "make_layer_edge_inputs_torch",
           "make_gdn_inputs", "make_gdn_inputs_torch",
           "f32_to_bf16_bits",
           "bf16_bits_to_f32", "random_addressing"]


@dataclasses.dataclass(frozen=True)
class Dims:
    B: int
    T: int
    H: int
    d_k: int
    n_sub: int
    d_v: int
    k_prime: int
    W: int
    R: int
    in_dtype: str = "bf16"          # "bf16" or "f32" for k, q, v and the codebooks

    @property
    def N(self) -> int:
        return self.n_sub * self.n_sub

    @property
    def half(self) -> int:
        return self.d_k // 2

    def replace(self, **kw) -> "Dims":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Preset:
    name: str
    dims: Dims
    reuse_frac: float = 0.0     # fraction of (b, t>=1, h) with k_t := k_{t-1}
    recall_frac: float = 0.0    # fraction of (b, t>=1, h) with q_t := k_s, s < t
    description: str = ""


PRESETS: Dict[str, Preset] = {
    "tiny": Preset("tiny", Dims(B=1, T=256, H=1, d_k=32, n_sub=32, d_v=32,
                                 k_prime=4, W=4, R=4, in_dtype="f32"),
                   description="tiny SDM layer, fp32 throughout, N=1024 slots"),
    "small": Preset("small", Dims(B=4, T=4096, H=8, d_k=128, n_sub=256, d_v=64,
                                   k_prime=16, W=16, R=16),
                    description="small layer, N=65,536 slots per head"),
    "prefill_1p4b": Preset("prefill_1p4b", Dims(B=8, T=8192, H=16, d_k=128, n_sub=512,
                                                 d_v=128, k_prime=32, W=32, R=32),
                           reuse_frac=0.05,
                           description="1.4B-scale layer prefill, N=262,144 slots per head, "
                                       "5% of tokens reuse the previous token's key"),
    "decode": Preset("decode", Dims(B=32, T=1024, H=8, d_k=128, n_sub=1024, d_v=128,
                                     k_prime=32, W=32, R=32),
                     description="decode: 32 sequences x 1024 single-token steps, "
                                 "N=1,048,576 slots per head"),
    "long_context": Preset("long_context", Dims(B=1, T=1 << 20, H=16, d_k=128, n_sub=1024,
                                                 d_v=128, k_prime=32, W=32, R=32),
                           recall_frac=0.01,
                           description="long-context prefill, 1M tokens, 1% of queries "
                                       "repeat an earlier key"),
}


def preset(name: str) -> Preset:
    return PRESETS[name]


# ---------------------------------------------------------------------------
# bf16 encoding (input quantisation only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if not np.isfinite(x).all():
        raise ValueError("bf16 encoding of non-finite inputs is not supported")
    bias = (u >> np.uint32(16)) & np.uint32(1)
    bias += np.uint32(0x7FFF)
    bias += u                       # finite fp32 bit patterns cannot overflow here
    return (bias >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-z.astype(np.float64)))).astype(np.float32)


# ---------------------------------------------------------------------------
# numpy backend
# ---------------------------------------------------------------------------
_STREAMS = ("C", "k", "q", "v", "a", "b", "M0", "masks")


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return {name: np.random.Generator(np.random.PCG64(s))
            for name, s in zip(_STREAMS, ss.spawn(len(_STREAMS)))}


def _normal(g: np.random.Generator, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def make_inputs(d: Dims, seed: int = 0, *, reuse_frac: float = 0.0, recall_frac: float = 0.0,
                m0: bool = True, separate_read_codebook: bool = False) -> dict:
    """Draw one batch of host inputs (numpy backend).

    Returns a dict with
      k, q   : [B,T,H,d_k]   uint16 bf16 bits (or float32 when d.in_dtype == "f32")
      v      : [B,T,H,d_v]   same encoding
      C_w    : [H,2,n_sub,d_k/2] same encoding; C_r is C_w unless separate_read_codebook
      a, b   : [B,T,H]       float32 gates
      M0     : [H,N,d_v]     float32 learned initial memory (if m0)
    """
    g = _streams(seed)
    half = d.d_k // 2
    C = _normal(g["C"], (H := d.H, 2, d.n_sub, half), std=1.0 / math.sqrt(half))
    C2 = _normal(g["C"], (H, 2, d.n_sub, half), std=1.0 / math.sqrt(half)) if separate_read_codebook else None
    k = _normal(g["k"], (d.B, d.T, d.H, d.d_k))
    q = _normal(g["q"], (d.B, d.T, d.H, d.d_k))
    v = _normal(g["v"], (d.B, d.T, d.H, d.d_v))
    a = _sigmoid(_normal(g["a"], (d.B, d.T, d.H), mean=3.0))
    b = _sigmoid(_normal(g["b"], (d.B, d.T, d.H)))
    M0 = _normal(g["M0"], (d.H, d.N, d.d_v), std=math.sqrt(0.02)) if m0 else None
    mg = g["masks"]
    if reuse_frac > 0 and d.T > 1:
        mask = mg.random((d.B, d.T, d.H)) < reuse_frac
        mask[:, 0, :] = False
        # k_t := k_{t-1} exactly; applied in token order so runs of reuse copy the same key
        for t in range(1, d.T):
            m = mask[:, t, :]
            if m.any():
                k[:, t, :, :][m] = k[:, t - 1, :, :][m]
    if recall_frac > 0 and d.T > 1:
        mask = mg.random((d.B, d.T, d.H)) < recall_frac
        mask[:, 0, :] = False
        bb, tt, hh = np.nonzero(mask)
        src = np.floor(mg.random(tt.shape) * tt).astype(np.int64)
        q[bb, tt, hh, :] = k[bb, src, hh, :]
    if d.in_dtype == "bf16":
        enc = f32_to_bf16_bits
    elif d.in_dtype == "f32":
        enc = lambda x: np.ascontiguousarray(x, dtype=np.float32)
    else:
        raise ValueError(d.in_dtype)
    out = dict(k=enc(k), q=enc(q), v=enc(v), C_w=enc(C), a=a, b=b)
    out["C_r"] = enc(C2) if C2 is not None else out["C_w"]
    if M0 is not None:
        out["M0"] = M0
    return out


def make_preset_inputs(name: str, seed: int = 0, **overrides) -> dict:
    p = PRESETS[name]
    d = p.dims.replace(**overrides) if overrides else p.dims
    return make_inputs(d, seed, reuse_frac=p.reuse_frac, recall_frac=p.recall_frac)


def make_inputs_torch(d: Dims, seed: int = 0, *, reuse_frac: float = 0.0, recall_frac: float = 0.0,
                      m0: bool = True, device: str = "cuda") -> dict:
    """Same tensors and distributions as make_inputs, drawn on the GPU with a
    seeded torch generator (for layers too large to draw on the host).
    Returns torch tensors on `device` (bf16 inputs as torch.bfloat16)."""
    import torch
    g = torch.Generator(device=device)
    half = d.d_k // 2
    dt = torch.bfloat16 if d.in_dtype == "bf16" else torch.float32

    def normal(shape, std=1.0, mean=0.0, sub=0):
        g.manual_seed(int(seed) * 1000003 + sub)
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        if mean != 0.0:
            x.add_(mean)
        return x

    out = {}
    out["C_w"] = normal((d.H, 2, d.n_sub, half), std=1.0 / math.sqrt(half), sub=1).to(dt)
    out["C_r"] = out["C_w"]
    k = normal((d.B, d.T, d.H, d.d_k), sub=2)
    q = normal((d.B, d.T, d.H, d.d_k), sub=3)
    out["v"] = normal((d.B, d.T, d.H, d.d_v), sub=4).to(dt)
    out["a"] = torch.sigmoid(normal((d.B, d.T, d.H), mean=3.0, sub=5))
    out["b"] = torch.sigmoid(normal((d.B, d.T, d.H), sub=6))
    if m0:
        out["M0"] = normal((d.H, d.N, d.d_v), std=math.sqrt(0.02), sub=7)
    g.manual_seed(int(seed) * 1000003 + 8)
    if reuse_frac > 0 and d.T > 1:
        mask = torch.rand((d.B, d.T, d.H), generator=g, device=device) < reuse_frac
        mask[:, 0, :] = False
        # k_t := k_{t-1}; a run of reuses copies the key at the run's start
        tidx = torch.arange(d.T, device=device).view(1, d.T, 1).expand(d.B, d.T, d.H)
        src = torch.where(mask, torch.zeros_like(tidx), tidx)
        src = torch.cummax(src, dim=1).values
        k = torch.gather(k, 1, src.unsqueeze(-1).expand(-1, -1, -1, d.d_k))
    if recall_frac > 0 and d.T > 1:
        mask = torch.rand((d.B, d.T, d.H), generator=g, device=device) < recall_frac
        mask[:, 0, :] = False
        bb, tt, hh = torch.nonzero(mask, as_tuple=True)
        srct = torch.floor(torch.rand(tt.shape, generator=g, device=device) * tt).long()
        q[bb, tt, hh, :] = k[bb, srct, hh, :]
    out["k"] = k.to(dt)
    out["q"] = q.to(dt)
    return out


def make_layer_edge_inputs(d: Dims, seed: int = 0) -> dict:
    """Inputs of the steps either side of the path (numpy backend).

      a_raw, b_raw : [B,T,H]        float32 gate pre-activations, N(0, 1)
      A            : [H]            float32 decay rates, U(0, 16)
      dt_bias      : [H]            float32 time-step bias, U(-6.9, -2.25) (the
                                    inverse softplus of a time step in [1e-3, 0.1])
      o            : [B,T,H,d_v]    float32 read-out, N(0, 0.5^2)
      g            : [B,T,H,d_v]    output-gate pre-activation N(0, 1), bf16 bits
                                    (or float32 when d.in_dtype == "f32")
      gamma        : [d_v]          float32 norm gain, 1 + N(0, 0.1^2)
    Drawn from sub-streams of their own, so the other inputs of a seed do not change.
    """
    names = ("a_raw", "b_raw", "A", "dt_bias", "o", "g", "gamma")
    ss = np.random.SeedSequence([seed, 104729])
    gs = {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(names, ss.spawn(len(names)))}
    shp = (d.B, d.T, d.H)
    g = _normal(gs["g"], shp + (d.d_v,))
    return dict(a_raw=_normal(gs["a_raw"], shp), b_raw=_normal(gs["b_raw"], shp),
                A=gs["A"].uniform(0.0, 16.0, d.H).astype(np.float32),
                dt_bias=gs["dt_bias"].uniform(-6.9, -2.25, d.H).astype(np.float32),
                o=_normal(gs["o"], shp + (d.d_v,), std=0.5),
                g=f32_to_bf16_bits(g) if d.in_dtype == "bf16" else g,
                gamma=_normal(gs["gamma"], (d.d_v,), std=0.1, mean=1.0))


def make_layer_edge_grads(d: Dims, seed: int = 0) -> dict:
    """Upstream gradients for the backward of the steps either side of the
    path (numpy backend), all float32 N(0, 1):
      da, db : [B,T,H]      dL/da and dL/db (what the scan's backward gives)
      dy     : [B,T,H,d_v]  dL/dy (what the head-mixing projection's backward gives)
    """
    names = ("da", "db", "dy")
    ss = np.random.SeedSequence([seed, 611953])
    gs = {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(names, ss.spawn(len(names)))}
    shp = (d.B, d.T, d.H)
    return dict(da=_normal(gs["da"], shp), db=_normal(gs["db"], shp), dy=_normal(gs["dy"], shp + (d.d_v,)))


def make_layer_edge_inputs_torch(d: Dims, seed: int = 0, device: str = "cuda") -> dict:
    """The distributions of make_layer_edge_inputs drawn on the GPU (torch
    generator; for layers too large to draw on the host)."""
    import torch
    gen = torch.Generator(device=device)
    dt = torch.bfloat16 if d.in_dtype == "bf16" else torch.float32
    shp = (d.B, d.T, d.H)

    def draw(sub, shape, kind="normal"):
        gen.manual_seed(int(seed) * 1000003 + 100 + sub)
        f = torch.randn if kind == "normal" else torch.rand
        return f(shape, generator=gen, device=device, dtype=torch.float32)

    return dict(a_raw=draw(0, shp), b_raw=draw(1, shp), A=draw(2, (d.H,), "uniform") * 16.0,
                dt_bias=draw(3, (d.H,), "uniform") * 4.65 - 6.9, o=draw(4, shp + (d.d_v,)) * 0.5,
                g=draw(5, shp + (d.d_v,)).to(dt), gamma=draw(6, (d.d_v,)) * 0.1 + 1.0)


def make_gdn_inputs(d: Dims, seed: int = 0) -> dict:
    """Inputs of the dense Gated DeltaNet recurrence (numpy backend).

      k, q : [B,T,H,d_k]   unit-norm directions (N(0,1) draws scaled to length 1,
                           as Gated DeltaNet normalises its keys and queries),
                           bf16 bits (or float32 when d.in_dtype == "f32")
      v    : [B,T,H,d_v]   N(0,1), same encoding
      a, b : [B,T,H]       float32, sigmoid(N(3,1)) and sigmoid(N(0,1)) as for SDM
      S0   : [B,H,d_k,d_v] float32 initial state, N(0, 0.02) (variance)
    """
    names = ("k", "q", "v", "a", "b", "S0")
    ss = np.random.SeedSequence([seed, 130363])
    gs = {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(names, ss.spawn(len(names)))}
    shp = (d.B, d.T, d.H)

    def unit(g):
        x = _normal(g, shp + (d.d_k,)).astype(np.float64)
        x /= np.maximum(np.linalg.norm(x, axis=-1, keepdims=True), 1e-30)
        return x.astype(np.float32)

    enc = f32_to_bf16_bits if d.in_dtype == "bf16" else (lambda x: np.ascontiguousarray(x, np.float32))
    return dict(k=enc(unit(gs["k"])), q=enc(unit(gs["q"])), v=enc(_normal(gs["v"], shp + (d.d_v,))),
                a=_sigmoid(_normal(gs["a"], shp, mean=3.0)), b=_sigmoid(_normal(gs["b"], shp)),
                S0=_normal(gs["S0"], (d.B, d.H, d.d_k, d.d_v), std=math.sqrt(0.02)))


def make_gdn_inputs_torch(d: Dims, seed: int = 0, device: str = "cuda") -> dict:
    """The distributions of make_gdn_inputs drawn on the GPU (torch generator)."""
    import torch
    gen = torch.Generator(device=device)
    dt = torch.bfloat16 if d.in_dtype == "bf16" else torch.float32
    shp = (d.B, d.T, d.H)

    def normal(sub, shape):
        gen.manual_seed(int(seed) * 1000003 + 200 + sub)
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)

    def unit(sub):
        x = normal(sub, shp + (d.d_k,))
        return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)

    return dict(k=unit(0).to(dt), q=unit(1).to(dt), v=normal(2, shp + (d.d_v,)).to(dt),
                a=torch.sigmoid(normal(3, shp) + 3.0), b=torch.sigmoid(normal(4, shp)),
                S0=normal(5, (d.B, d.H, d.d_k, d.d_v)) * math.sqrt(0.02))


def random_addressing(d: Dims, seed: int = 0, *, hazard_slots: Optional[int] = None) -> dict:
    """Random (not PKM-derived) slot lists and weights for scan-only tests.

    Each token gets W distinct write slots and R distinct read slots drawn
    uniformly from [0, N) (or from [0, hazard_slots) to force frequent
    collisions between tokens), and positive weights that sum to one per list.
    """
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7919])))
    pool = d.N if hazard_slots is None else min(hazard_slots, d.N)
    if pool < max(d.W, d.R):
        raise ValueError("slot pool smaller than the list length")

    def lists(n):
        shape = (d.B, d.T, d.H, n)
        if pool <= 4096:
            # distinct slots per list: argsort of random keys over the whole pool
            keys = g.random((d.B, d.T, d.H, pool))
            return np.argsort(keys, axis=-1)[..., :n].astype(np.int32)
        # large pool: draw, then redraw any list that holds a repeated slot
        x = g.integers(0, pool, size=shape, dtype=np.int64).reshape(-1, n)
        while True:
            srt = np.sort(x, axis=1)
            bad = np.nonzero((srt[:, 1:] == srt[:, :-1]).any(axis=1))[0]
            if bad.size == 0:
                break
            x[bad] = g.integers(0, pool, size=(bad.size, n), dtype=np.int64)
        return x.reshape(shape).astype(np.int32)

    def weights(n):
        w = g.random((d.B, d.T, d.H, n)).astype(np.float64) + 0.05
        return (w / w.sum(-1, keepdims=True)).astype(np.float32)

    return dict(widx=lists(d.W), wwt=weights(d.W), ridx=lists(d.R), rwt=weights(d.R))
