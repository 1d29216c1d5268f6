"""Seeded synthetic workloads for the int4 KV-cache decode path.

This module only draws random numbers: it holds none of the method's
arithmetic (no quantisation, no attention).  Both the HIP path and the CPU
oracle receive the tensors it returns (the oracle gets the exact fp16 bytes,
copied to the host), so the two sides never depend on generator parity.

The shapes follow the model shapes the FlexGen pages evaluate on (OPT-6.7B,
OPT-30B, OPT-175B with prompt length 512 and 32 generated tokens; effective
batch 144 for the 4-bit OPT-175B run -- "FlexGen研究学术报告", section 四.1) and
the decode-phase notation of the FlexGen blog (b, a, h, s, n; section
"P/D阶段计算").  No dataset, prompt or trained weight is used: every
activation is a seeded normal draw.

Layouts handed to the library:
  prefill Q/K/V    fp16 [b][s][a][d]   (the blog's [b, s, a, h/a] cache shape)
  q, k_new, v_new  fp16 [b][1][a][d]
"""
from __future__ import annotations

import dataclasses
import math

import torch

# tensor ids used in the seed formula
TID_K, TID_V, TID_Q, TID_KNEW, TID_VNEW = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    idx: int            # config number, part of every seed
    b: int              # (effective) batch
    a: int              # heads
    d: int              # head_dim = h / a
    s: int              # prompt length
    n: int              # decode steps
    layers: int         # layers whose caches stay resident
    std: float = 1.0    # N(0, std^2) for q, k, v
    outlier_frac: float = 0.0   # fraction of the h channels multiplied by outlier_mult
    outlier_mult: float = 1.0
    boost_frac: float = 0.0     # fraction of key positions per (b, a) multiplied by boost_mult
    boost_mult: float = 1.0
    topk_frac: float = 0.0      # > 0: the sparse variant keeps ceil(topk_frac * T) keys

    @property
    def h(self) -> int:
        return self.a * self.d

    @property
    def S(self) -> int:
        """Cache capacity in token slots: prompt + generated."""
        return self.s + self.n

    def k_top(self, T: int) -> int:
        return max(1, math.ceil(self.topk_frac * T - 1e-9))


TINY = Workload("tiny", 1, b=2, a=2, d=64, s=16, n=4, layers=1)
OPT_6_7B = Workload("opt-6.7b", 2, b=32, a=32, d=128, s=512, n=32, layers=32, std=0.5)
OPT_30B = Workload("opt-30b", 3, b=256, a=56, d=128, s=512, n=32, layers=48,
                   outlier_frac=0.01, outlier_mult=8.0)
OPT_175B = Workload("opt-175b", 4, b=144, a=96, d=128, s=512, n=32, layers=96)
SPARSE = Workload("sparse-top10", 5, b=32, a=96, d=128, s=2047, n=1, layers=1,
                  boost_frac=0.05, boost_mult=3.0, topk_frac=0.10)

ALL = (TINY, OPT_6_7B, OPT_30B, OPT_175B, SPARSE)
BY_NAME = {w.name: w for w in ALL}


def seed_of(w: Workload, layer: int, step: int, tid: int) -> int:
    """Distinct seed per (config, layer, step, tensor); step 0 = prefill, j = decode step j."""
    return ((100 * w.idx + layer) * 100 + step) * 8 + tid


def _normal(shape, seed: int, device, std: float) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def outlier_channels(w: Workload, device="cpu") -> torch.Tensor | None:
    """Seeded set of outlier channels among the h = a*d channels (same for all b, t, layers)."""
    if w.outlier_frac <= 0:
        return None
    n_out = max(1, round(w.outlier_frac * w.h))
    g = torch.Generator(device="cpu")
    g.manual_seed(1_000_003 * w.idx + 17)
    return torch.randperm(w.h, generator=g)[:n_out].to(device)


def _apply_outliers(x: torch.Tensor, w: Workload) -> torch.Tensor:
    ch = outlier_channels(w, x.device)
    if ch is None:
        return x
    flat = x.view(*x.shape[:-2], w.h)
    flat[..., ch] *= w.outlier_mult
    return x


def prefill_kv(w: Workload, layer: int, device, s_len: int | None = None, b: int | None = None):
    """Prompt K and V, fp16 [b][s_len][a][d]."""
    s_len = w.s if s_len is None else s_len
    b = w.b if b is None else b
    out = []
    for tid in (TID_K, TID_V):
        x = _normal((b, s_len, w.a, w.d), seed_of(w, layer, 0, tid), device, w.std)
        x = _apply_outliers(x, w)
        if tid == TID_K and w.boost_frac > 0:
            x = _boost_positions(x, w, layer, device)
        out.append(x.half())
    return out[0], out[1]


def prefill_q(w: Workload, layer: int, device, s_len: int | None = None, b: int | None = None) -> torch.Tensor:
    """Prompt queries for the prefill attention, fp16 [b][s_len][a][d] (same distribution
    and outlier channels as q of the decode steps)."""
    s_len = w.s if s_len is None else s_len
    b = w.b if b is None else b
    x = _normal((b, s_len, w.a, w.d), seed_of(w, layer, 0, TID_Q), device, w.std)
    return _apply_outliers(x, w).half()


def _boost_positions(k: torch.Tensor, w: Workload, layer: int, device) -> torch.Tensor:
    """Multiply a seeded random boost_frac of the token positions of every (b, a) by boost_mult."""
    b, s_len, a, _ = k.shape
    n_boost = max(1, int(w.boost_frac * s_len))
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(w, layer, 0, 7))
    r = torch.rand((b, a, s_len), generator=g, device=device)
    pos = r.topk(n_boost, dim=-1).indices                      # [b][a][n_boost]
    mult = torch.ones((b, a, s_len), device=device)
    mult.scatter_(-1, pos, w.boost_mult)
    return k * mult.permute(0, 2, 1).unsqueeze(-1)


def decode_inputs(w: Workload, layer: int, step: int, device, b: int | None = None):
    """Decode step `step` (1-based): q, k_new, v_new, each fp16 [b][1][a][d]."""
    b = w.b if b is None else b
    out = []
    for tid in (TID_Q, TID_KNEW, TID_VNEW):
        x = _normal((b, 1, w.a, w.d), seed_of(w, layer, step, tid), device, w.std)
        x = _apply_outliers(x, w)
        if tid == TID_KNEW and w.boost_frac > 0:
            g = torch.Generator(device=device)
            g.manual_seed(seed_of(w, layer, step, 7))
            sel = torch.rand((b, 1, w.a, 1), generator=g, device=device) < w.boost_frac
            x = torch.where(sel, x * w.boost_mult, x)
        out.append(x.half())
    return out[0], out[1], out[2]


def random_fp16(shape, seed: int, device="cpu", std: float = 1.0) -> torch.Tensor:
    """Generic seeded N(0, std^2) fp16 tensor (edge-case tests)."""
    return _normal(shape, seed, device, std).half()
