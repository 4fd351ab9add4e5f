"""Seeded synthetic MoE-layer inputs, shared by the oracle tests, the GPU tests and bench.py.

This module only draws random numbers and lays them out. It holds none of the MoE layer's
arithmetic (no routing, no grouping, no GEMM, no combine): the oracle and the HIP library
both consume exactly the tensors produced here.

Recipe (one generator per tensor, in a fixed order, all derived from one integer seed):

* router scores  fp32 [T, E]
    - "normal":  N(0, 1), rows redrawn until all E values of the row are distinct
    - "uniform": U[0, 1)
    - "zipf":    U[0, 1) + log p_e, where p_e = (1/rank_e) / sum_{r<=E} 1/r and rank is
                 1 + a seeded random permutation of the experts (Zipf exponent 1.0)
* activations    bf16 [T, H], N(0, 1) drawn in fp32 and rounded to bf16 (round-to-nearest-even)
* expert weights per expert (routed experts 0..E-1, then the shared expert): gate [I, H],
  up [I, H], down [H, I] in nn.Linear layout (output rows, input contiguous), N(0, 0.02^2)
    - "bf16": rounded to bf16
    - "fp8":  quantised per 128x128 block: s = amax(|w|)/448 (s = 1 if the block is all zero),
              q = e4m3fn(clamp(w / s, -448, 448)) with round-to-nearest-even; the stored fp32
              scale multiplies: w ~= q * s

The MoE shapes follow DeepSeek-V3 (256 routed experts of three 7168x2048 matrices, top-8,
one shared expert) and Kimi-K2 (384 experts of the same shape), as the pages describe them.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

BLOCK = 128  # side of the fp32 scale block of FP8 weights

# name -> shape/recipe.  T tokens, H hidden, I expert intermediate, E routed experts, k top-k.
CONFIGS = {
    # 16 routed experts + 1 shared, top-2 softmax, bf16 weights (small case, fits the oracle)
    "tiny": dict(T=16, H=256, I=128, E=16, k=2, score_fn="softmax", scores="normal", wdtype="bf16"),
    # the tiny layer with FP8 block-quantised weights (exercises the FP8 path at tiny size)
    "tiny_fp8": dict(T=16, H=256, I=128, E=16, k=2, score_fn="softmax", scores="normal", wdtype="fp8"),
    # DeepSeek-V3-shaped layer, decode batch of 16 tokens
    "dsv3_decode": dict(T=16, H=7168, I=2048, E=256, k=8, score_fn="sigmoid", scores="uniform", wdtype="fp8"),
    # DeepSeek-V3-shaped layer, 4096-token prefill
    "dsv3_prefill": dict(T=4096, H=7168, I=2048, E=256, k=8, score_fn="sigmoid", scores="uniform", wdtype="fp8"),
    # DeepSeek-V3-shaped layer, 32768-token prefill with Zipf-skewed expert popularity
    "dsv3_long_zipf": dict(T=32768, H=7168, I=2048, E=256, k=8, score_fn="sigmoid", scores="zipf", wdtype="fp8"),
    # Kimi-K2-shaped layer, 8192-token prefill, 384 experts
    "kimi_k2": dict(T=8192, H=7168, I=2048, E=384, k=8, score_fn="sigmoid", scores="uniform", wdtype="fp8"),
}


@dataclasses.dataclass
class ExpertWeights:
    """Weights of n experts. fp8: uint8 codes + fp32 scales; bf16: uint16 bit patterns; mxfp4:
    uint8 bytes of two FP4 codes [n, rows, cols/2] + E8M0 bytes [n, rows, cols/32]."""

    wdtype: str  # "fp8", "bf16" or "mxfp4"
    gate: torch.Tensor  # [n, I, H]
    up: torch.Tensor  # [n, I, H]
    down: torch.Tensor  # [n, H, I]
    s_gate: torch.Tensor | None  # [n, I/128, H/128] fp32
    s_up: torch.Tensor | None
    s_down: torch.Tensor | None  # [n, H/128, I/128]

    @property
    def n(self) -> int:
        return self.gate.shape[0]

    def to(self, device) -> "ExpertWeights":
        f = lambda t: None if t is None else t.to(device)
        return ExpertWeights(self.wdtype, f(self.gate), f(self.up), f(self.down),
                             f(self.s_gate), f(self.s_up), f(self.s_down))

    def select(self, idx) -> "ExpertWeights":
        """Experts idx (a list of ints), copied to host memory."""
        ii = torch.as_tensor(list(idx), dtype=torch.long, device=self.gate.device)
        f = lambda t: None if t is None else t.index_select(0, ii).cpu().contiguous()
        return ExpertWeights(self.wdtype, f(self.gate), f(self.up), f(self.down),
                             f(self.s_gate), f(self.s_up), f(self.s_down))


@dataclasses.dataclass
class Layer:
    T: int
    H: int
    I: int
    E: int
    k: int
    score_fn: str  # "softmax" or "sigmoid"
    renorm: int
    scores: torch.Tensor  # fp32 [T, E]
    x: torch.Tensor  # uint16 bf16 bits [T, H]  (torch.int16 storage viewed as bits)
    experts: ExpertWeights  # E routed experts
    shared: ExpertWeights  # 1 shared expert

    def to(self, device) -> "Layer":
        return dataclasses.replace(self, scores=self.scores.to(device), x=self.x.to(device),
                                   experts=self.experts.to(device), shared=self.shared.to(device))


def _seed(seed: int, *stream: int) -> int:
    """A 63-bit seed for one tensor stream, derived from (seed, stream ids) with SeedSequence."""
    ss = np.random.SeedSequence([seed, *stream])
    return int(ss.generate_state(2, dtype=np.uint32).astype(np.uint64) @ np.array([1, 1 << 31], dtype=np.uint64)) & ((1 << 63) - 1)


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """fp32 tensor -> bf16 (RNE, torch's cast) -> raw 16-bit patterns as torch.int16."""
    return t.to(torch.bfloat16).view(torch.int16)


def _router_scores(kind: str, T: int, E: int, seed: int) -> torch.Tensor:
    rng = np.random.default_rng(_seed(seed, 1))
    if kind == "normal":
        s = rng.standard_normal((T, E), dtype=np.float32)
        for t in range(T):
            while len(np.unique(s[t])) != E:
                s[t] = rng.standard_normal(E, dtype=np.float32)
    elif kind == "uniform":
        s = rng.random((T, E), dtype=np.float32)
    elif kind == "zipf":
        u = rng.random((T, E), dtype=np.float32)
        rank = 1 + np.random.default_rng(_seed(seed, 5)).permutation(E)
        harmonic = np.sum(1.0 / np.arange(1, E + 1, dtype=np.float64))
        logp = np.log((1.0 / rank) / harmonic)
        s = (u.astype(np.float64) + logp[None, :]).astype(np.float32)
    else:
        raise ValueError(kind)
    return torch.from_numpy(np.ascontiguousarray(s))


def _activations(T: int, H: int, seed: int) -> torch.Tensor:
    rng = np.random.default_rng(_seed(seed, 2))
    return bf16_bits(torch.from_numpy(rng.standard_normal((T, H), dtype=np.float32)))


def quantize_fp8_blocks(w: torch.Tensor):
    """Per-128x128-block e4m3fn quantisation of w [..., N, K] (fp32): returns (codes uint8, scales fp32)."""
    *lead, N, K = w.shape
    assert N % BLOCK == 0 and K % BLOCK == 0, (N, K)
    wb = w.reshape(*lead, N // BLOCK, BLOCK, K // BLOCK, BLOCK)
    amax = wb.abs().amax(dim=(-3, -1))  # [..., N/128, K/128]
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    q = (wb / s[..., :, None, :, None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(*lead, N, K).contiguous(), s.contiguous()


MX_GROUP = 32  # values along K sharing one E8M0 scale in the 4-bit weight format


def quantize_mxfp4(w: torch.Tensor):
    """OCP microscaling FP4 quantisation of w [..., N, K] (fp32) along K: per group of 32 the
    shared scale 2^X with X = floor(log2(max|w|)) - 2 (E8M0 byte X + 127; 0 for an all-zero
    group), elements = E2M1 of w / 2^X rounded to nearest even and saturated at 6.  Returns
    (packed codes uint8 [..., N, K/2]: element 2j in the low nibble of byte j, E8M0 bytes uint8
    [..., N, K/32])."""
    *lead, N, K = w.shape
    assert K % MX_GROUP == 0, K
    g = w.reshape(*lead, N, K // MX_GROUP, MX_GROUP)
    amax = g.abs().amax(dim=-1)
    X = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 2, torch.full_like(amax, -127.0))
    X = X.clamp(-127, 127)
    p = (g / torch.exp2(X)[..., None]).abs()
    # E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); ties go to the even code
    edges = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], device=w.device)
    idx = torch.bucketize(p, edges, right=False)  # a value on an edge gets the lower code
    tie = torch.isin(p, edges)
    idx = torch.where(tie & (idx % 2 == 1), idx + 1, idx)  # ties go to the even code
    codes = (idx | torch.where(g < 0, 8, 0)).to(torch.uint8).reshape(*lead, N, K)
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    return packed.contiguous(), (X + 127).to(torch.uint8).contiguous()


CHUNK = 16  # experts drawn per generator call


def _expert_weights(n: int, H: int, I: int, wdtype: str, seed: int, stream0: int, device) -> ExpertWeights:
    """n experts, drawn in chunks of CHUNK experts: chunk c draws its gate, up and down tensors
    [m, rows, cols] from streams (stream0 + c, 0..2)."""
    gate, up, down, sg, su, sd = [], [], [], [], [], []
    for c0 in range(0, n, CHUNK):
        m_ = min(CHUNK, n - c0)
        mats = []
        for m, shape in enumerate(((I, H), (I, H), (H, I))):
            g = torch.Generator(device=device)
            g.manual_seed(_seed(seed, stream0 + c0, m))
            w = torch.randn((m_, *shape), generator=g, device=device, dtype=torch.float32) * 0.02
            mats.append(w)
        if wdtype == "fp8":
            (qg, s_g), (qu, s_u), (qd, s_d) = (quantize_fp8_blocks(w) for w in mats)
            gate.append(qg); up.append(qu); down.append(qd); sg.append(s_g); su.append(s_u); sd.append(s_d)
        elif wdtype == "mxfp4":
            (qg, s_g), (qu, s_u), (qd, s_d) = (quantize_mxfp4(w) for w in mats)
            gate.append(qg); up.append(qu); down.append(qd); sg.append(s_g); su.append(s_u); sd.append(s_d)
        elif wdtype == "bf16":
            gate.append(bf16_bits(mats[0])); up.append(bf16_bits(mats[1])); down.append(bf16_bits(mats[2]))
        else:
            raise ValueError(wdtype)
        del mats
    st = lambda xs: torch.cat(xs).contiguous() if xs else None
    return ExpertWeights(wdtype, st(gate), st(up), st(down), st(sg), st(su), st(sd))


def make_layer(cfg: str | dict, seed: int = 0, device="cpu", **overrides) -> Layer:
    """Build a seeded synthetic layer. `cfg` is a CONFIGS name or a dict with the same keys.

    Router scores and activations are drawn with numpy on the host (then moved to `device`);
    the expert weights are drawn with torch's generator on `device` (large layers are drawn
    on the GPU for speed), so a layer is reproducible for a given (seed, device kind).
    """
    c = dict(CONFIGS[cfg]) if isinstance(cfg, str) else dict(cfg)
    c.update(overrides)
    T, H, I, E, k = c["T"], c["H"], c["I"], c["E"], c["k"]
    scores = _router_scores(c.get("scores", "uniform"), T, E, seed)
    x = _activations(T, H, seed)
    experts = _expert_weights(E, H, I, c["wdtype"], seed, 1000, device)
    shared = _expert_weights(1, H, I, c["wdtype"], seed, 1000 + E, device)
    return Layer(T=T, H=H, I=I, E=E, k=k, score_fn=c["score_fn"], renorm=int(c.get("renorm", 1)),
                 scores=scores.to(device), x=x.to(device), experts=experts, shared=shared)


def random_topk_ids(T: int, E: int, k: int, seed: int, skew: float = 0.0) -> torch.Tensor:
    """int32 [T, k]: k distinct experts per row; skew > 0 concentrates rows on low expert ids."""
    rng = np.random.default_rng(_seed(seed, 7))
    ids = np.empty((T, k), dtype=np.int32)
    p = None
    if skew > 0:
        p = 1.0 / np.arange(1, E + 1) ** skew
        p = p / p.sum()
    for t in range(T):
        ids[t] = rng.choice(E, size=k, replace=False, p=p)
    return torch.from_numpy(ids)


def random_fp8_activations(rows: int, K: int, seed: int, exp_range=(-8, 8)):
    """Quantised activations drawn directly: (codes uint8 [rows, K], every finite E4M3FN code
    (the NaN codes 0x7F and 0xFF excluded) equally likely; exps int8 [rows, K/128], block
    exponents uniform in exp_range)."""
    rng = np.random.default_rng(_seed(seed, 11))
    codes = rng.integers(0, 254, size=(rows, K), dtype=np.int64)
    codes = codes + (codes >= 0x7F)  # skip 0x7F; 0xFF is beyond the range drawn
    exps = rng.integers(exp_range[0], exp_range[1] + 1, size=(rows, K // 128))
    return torch.from_numpy(codes.astype(np.uint8)), torch.from_numpy(exps.astype(np.int8))
