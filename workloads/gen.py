"""Seeded synthetic workloads shaped like the expert layers the pages discuss.

Sources for the shapes and routing structure:
  * "Boosting MoE Training Throughput with Advanced Fusion Kernels" (NVIDIA
    technical blog, zh-cn translation): DeepSeek-V3 and GPT-OSS pretraining
    are the workloads it reports (§ "From kernel-level gains to pretraining
    speedups").
  * "NVIDIA Transformer Engine 优化 MoE 生物基础模型训练" (TE + BioNeMo Mixtral
    tutorial): Mixtral-8x7B with a top-2-of-8 router (Fig. 1, Fig. 5).

No dataset or trained weight is used: every tensor is drawn from a seeded
numpy generator. bf16 tensors are returned as uint16 bit patterns (numpy has
no bf16 dtype); they are rounded from float32 with torch's CPU cast
(round-to-nearest-even), so the same bits go to the GPU and to the oracle.

Sub-seed convention: base seed s; X uses s+1, W1 s+2, W2 s+3, router
logits / group sizes s+4, dOut s+5.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# --------------------------------------------------------------------------
# Workload descriptions.  `routing` picks how expert_idx / probs are drawn:
#   "softmax_topk": logits ~ N(0, sigma^2) i.i.d., softmax over all experts in
#                   fp32, keep the k largest (no renormalisation, ties to the
#                   lower expert id, slots in descending probability).
#   "biased_topk" : logits[t, e] = mu_e + eps[t, e], mu_e ~ N(0, var), eps ~
#                   N(0, 1): a persistent per-expert bias gives strong load
#                   imbalance (GPT-OSS-shaped layer).
#   "zipf"        : rows arrive already dispatched to this GPU's experts
#                   (k = 1 per row); group sizes are multinomial over
#                   Zipf(s)-weighted experts with some groups forced empty
#                   (DeepSeek-V3-shaped one-GPU share).
# --------------------------------------------------------------------------
CONFIGS = {
    "tiny": dict(E=4, k=2, T=256, H=128, I=256, routing="softmax_topk",
                 logit_sigma=1.0, act="swiglu", beta=1.0, clamp=None,
                 prec="bf16"),
    "mixtral": dict(E=8, k=2, T=8192, H=4096, I=14336, routing="softmax_topk",
                    logit_sigma=1.0, act="swiglu", beta=1.0, clamp=None,
                    prec="bf16"),
    "mixtral_mx": dict(E=8, k=2, T=8192, H=4096, I=14336,
                       routing="softmax_topk", logit_sigma=1.0, act="swiglu",
                       beta=1.0, clamp=None, prec="mxfp8"),
    "dsv3": dict(E=32, k=1, T=16384, H=7168, I=2048, routing="zipf",
                 zipf_s=1.2, n_empty=4, act="swiglu", beta=1.0, clamp=None,
                 prec="bf16"),
    "gptoss": dict(E=128, k=4, T=16384, H=2880, I=2880, routing="biased_topk",
                   logit_var=2.0, act="swiglu", beta=1.702, clamp=7.0,
                   prec="mxfp8"),
}

W_SIGMA = 0.02  # weights ~ N(0, 0.02^2)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns (torch CPU cast, RNE)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32)


def _normal_bf16(rng: np.random.Generator, shape, sigma: float,
                 chunk: int = 1 << 24) -> np.ndarray:
    """N(0, sigma^2) samples rounded to bf16, drawn in chunks to bound RAM."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = rng.standard_normal(e - s, dtype=np.float32)
        if sigma != 1.0:
            v *= np.float32(sigma)
        out[s:e] = bf16_bits_from_f32(v)
    return out.reshape(shape)


def _softmax_topk(logits: np.ndarray, k: int):
    """fp32 softmax over experts, then the k largest (ties -> lower id)."""
    lg = logits.astype(np.float32)
    m = lg.max(axis=1, keepdims=True)
    ex = np.exp(lg - m, dtype=np.float32)
    p = ex / ex.sum(axis=1, keepdims=True, dtype=np.float32)
    # stable argsort on -p keeps the lower expert id first among ties
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]
    probs = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return order.astype(np.int32), probs


def route_inputs(cfg: dict, seed: int, T: int, E: int, k: int):
    """Draw (expert_idx[T][k] int32, probs[T][k] float32) for a config."""
    rng = np.random.default_rng(seed + 4)
    kind = cfg["routing"]
    if kind == "softmax_topk":
        logits = rng.standard_normal((T, E), dtype=np.float32)
        logits *= np.float32(cfg.get("logit_sigma", 1.0))
        return _softmax_topk(logits, k)
    if kind == "biased_topk":
        mu = rng.standard_normal(E) * np.sqrt(cfg.get("logit_var", 2.0))
        eps = rng.standard_normal((T, E))
        return _softmax_topk((mu[None, :] + eps).astype(np.float32), k)
    if kind == "zipf":
        assert k == 1
        n_empty = min(cfg.get("n_empty", 4), E)
        empty = {0, E - 1}
        others = [e for e in rng.permutation(E).tolist() if e not in empty]
        empty.update(others[: max(0, n_empty - len(empty))])
        live = [e for e in range(E) if e not in empty]
        ranks = rng.permutation(len(live)) + 1
        w = ranks.astype(np.float64) ** (-cfg.get("zipf_s", 1.2))
        counts = rng.multinomial(T, w / w.sum())
        idx = np.repeat(np.asarray(live, dtype=np.int32), counts)
        idx = idx[rng.permutation(T)]
        probs = rng.uniform(0.0, 0.25, size=T).astype(np.float32)
        return idx.reshape(T, 1), probs.reshape(T, 1)
    raise ValueError(f"unknown routing kind {kind!r}")


@dataclasses.dataclass
class Workload:
    name: str
    E: int
    k: int
    T: int
    H: int
    I: int
    act: str
    beta: float
    clamp: Optional[float]
    prec: str
    seed: int
    expert_idx: np.ndarray          # int32 [T][k] global expert ids
    probs: np.ndarray               # float32 [T][k]
    x: Optional[np.ndarray] = None  # uint16 bf16 [T][H]
    w1: Optional[np.ndarray] = None  # uint16 bf16 [E][2I][H], rows gate|up
    w2: Optional[np.ndarray] = None  # uint16 bf16 [E][H][I]
    dout: Optional[np.ndarray] = None  # uint16 bf16 [T][H]
    first_expert: int = 0

    @property
    def M(self) -> int:
        """Routed rows that land on this GPU's experts."""
        e = self.expert_idx
        loc = (e >= self.first_expert) & (e < self.first_expert + self.E)
        return int(loc.sum())

    def m_cap(self, align: int = 128) -> int:
        """A row allocation that always fits the padded grouped layout."""
        return self.T * self.k + self.E * (align - 1)

    def group_sizes(self) -> np.ndarray:
        e = self.expert_idx.reshape(-1) - self.first_expert
        e = e[(e >= 0) & (e < self.E)]
        return np.bincount(e, minlength=self.E)


def make_workload(name: str, seed: int = 0, *, with_weights: bool = True,
                  with_acts: bool = True, w_sigma: float = W_SIGMA,
                  **overrides) -> Workload:
    """Build a seeded workload.  `overrides` may change E, k, T, H, I, act,
    beta, clamp, prec or routing parameters (smaller parity cases keep the
    routing structure of the named config)."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    E, k, T, H, I = (int(cfg[n]) for n in ("E", "k", "T", "H", "I"))
    idx, probs = route_inputs(cfg, seed, T, E, k)
    wl = Workload(name=name, E=E, k=k, T=T, H=H, I=I, act=cfg["act"],
                  beta=float(cfg["beta"]), clamp=cfg["clamp"],
                  prec=cfg["prec"], seed=seed, expert_idx=idx, probs=probs)
    if with_acts:
        wl.x = _normal_bf16(np.random.default_rng(seed + 1), (T, H), 1.0)
        wl.dout = _normal_bf16(np.random.default_rng(seed + 5), (T, H), 1.0)
    if with_weights:
        n1 = 2 * I if cfg["act"] != "srelu" else I
        wl.w1 = _normal_bf16(np.random.default_rng(seed + 2), (E, n1, H),
                             w_sigma)
        wl.w2 = _normal_bf16(np.random.default_rng(seed + 3), (E, H, I),
                             w_sigma)
    return wl
