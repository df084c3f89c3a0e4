"""Seeded synthetic inputs for EFLA workloads.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic.  The same tensors feed the HIP path and the fp64 oracle
(which receives them upcast from the exact bf16 / fp32 values).

The pages evaluate on language-model, sequential-MNIST and MAD suites that are
not reproduced here; these synthetic tensors stand in for one attention layer
at the 340M and 1.3B model shapes, plus a stiff long-context case that mimics
the "large key norm / high-energy input" regime of the pages' Problem section.

Layouts: q, k [B, L, H, dk]; v [B, L, H, dv]; beta [B, L, H];
s0 [B, H, dk, dv] float32 (or None).  Decode inputs carry a leading step axis:
q, k [steps, N, H, dk], v [steps, N, H, dv], beta [steps, N, H].  Packed
variable-length inputs: q, k [T, H, dk], v [T, H, dv], beta [T, H], int32
offsets cu_seqlens [N + 1], s0 [N, H, dk, dv].
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "get", "generate", "generate_decode", "generate_packed", "length_mix",
           "to_f64"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    dk: int
    dv: int
    chunk: int
    dtype: str            # "f32" or "bf16": dtype of q, k, v, beta and o
    qk: str               # "normal" | "unit" | "unit_u" (unit x U[0.5,2]) | "unit_logu_k"
    beta: str             # "sigmoid" (sigmoid(N(0,1))) | "u10" (U[0,10])
    s0: str               # "none" | "n002" (0.02 * N(0,1), float32)
    spikes: float = 0.0   # fraction of (b, t) positions whose v is scaled by 100
    seed: int = 0
    steps: int = 0        # decode workloads: consecutive single-token steps
    note: str = field(default="", compare=False)

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.L

    @property
    def tokens(self) -> int:
        return self.B * self.L


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 1, 1, 64, 16, 16, 16, "f32", "normal", "sigmoid", "none",
                 seed=1001, note="oracle-size case, unnormalised q/k (lambda ~ 16)"),
        Workload("small_bf16", 4, 8, 2048, 64, 64, 64, "bf16", "unit", "sigmoid", "none",
                 seed=1002, note="L2-normalised q/k"),
        Workload("shape_340m", 8, 8, 2048, 128, 128, 64, "bf16", "unit_u", "sigmoid", "n002",
                 seed=1003, note="340M-model-shaped layer"),
        Workload("shape_1p3b", 4, 16, 4096, 128, 128, 64, "bf16", "unit_u", "sigmoid", "n002",
                 seed=1004, note="1.3B-model-shaped layer"),
        Workload("stiff_64k", 1, 16, 65536, 128, 128, 64, "bf16", "unit_logu_k", "u10", "none",
                 spikes=0.05, seed=1005,
                 note="stiff long context: |k| log-uniform in [0.1, 30], beta ~ U[0,10], 5% x100 v spikes"),
        Workload("decode_1p3b", 256, 16, 1, 128, 128, 0, "bf16", "unit_u", "sigmoid", "n002",
                 seed=1014, steps=16, note="decode: 256 sequences x 16 heads, 16 single-token steps"),
        # B = number of sequences, L = total packed tokens (lengths from length_mix)
        Workload("varlen_1p3b", 16, 16, 16384, 128, 128, 64, "bf16", "unit_u", "sigmoid", "n002",
                 seed=1006, note="1.3B-shaped heads, 16 sequences of mixed length packed into 16384 tokens"),
    ]
}


def get(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def _torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def _cast(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    # float64 -> float32 -> target; float32 -> bfloat16 rounds to nearest even.
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(_torch_dtype(dtype)).to(device).contiguous()


def _directions(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    n[n == 0] = 1.0
    return x / n


def _qk(rng: np.random.Generator, shape, kind: str, is_key: bool) -> np.ndarray:
    if kind == "normal":
        return rng.standard_normal(shape)
    if kind == "unit":
        return _directions(rng, shape)
    if kind == "unit_u":
        return _directions(rng, shape) * rng.uniform(0.5, 2.0, size=shape[:-1] + (1,))
    if kind == "unit_logu_k":
        d = _directions(rng, shape)
        if is_key:
            r = np.exp(rng.uniform(np.log(0.1), np.log(30.0), size=shape[:-1] + (1,)))
        else:
            r = rng.uniform(0.5, 2.0, size=shape[:-1] + (1,))
        return d * r
    raise ValueError(kind)


def _beta(rng: np.random.Generator, shape, kind: str) -> np.ndarray:
    if kind == "sigmoid":
        return 1.0 / (1.0 + np.exp(-rng.standard_normal(shape)))
    if kind == "u10":
        return rng.uniform(0.0, 10.0, size=shape)
    raise ValueError(kind)


def generate(w: Workload, device="cpu", L: int | None = None, B: int | None = None,
             H: int | None = None, seed: int | None = None) -> dict:
    """Inputs for a chunked-forward workload (optionally resized)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    L = w.L if L is None else L
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = _qk(rng, (B, L, H, w.dk), w.qk, is_key=False)
    k = _qk(rng, (B, L, H, w.dk), w.qk, is_key=True)
    v = rng.standard_normal((B, L, H, w.dv))
    beta = _beta(rng, (B, L, H), w.beta)
    if w.spikes > 0:
        hit = rng.random((B, L)) < w.spikes
        v[hit] *= 100.0
    s0 = None
    if w.s0 == "n002":
        s0 = torch.from_numpy(0.02 * rng.standard_normal((B, H, w.dk, w.dv))).float().to(device)
    out = dict(q=_cast(q, w.dtype, device), k=_cast(k, w.dtype, device),
               v=_cast(v, w.dtype, device), beta=_cast(beta, w.dtype, device), s0=s0)
    return out


def generate_decode(w: Workload, device="cpu", N: int | None = None,
                    steps: int | None = None, seed: int | None = None) -> dict:
    """Inputs for a decode workload: per-step q, k, v, beta and the state s0."""
    N = w.B if N is None else N
    steps = w.steps if steps is None else steps
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = _qk(rng, (steps, N, w.H, w.dk), w.qk, is_key=False)
    k = _qk(rng, (steps, N, w.H, w.dk), w.qk, is_key=True)
    v = rng.standard_normal((steps, N, w.H, w.dv))
    beta = _beta(rng, (steps, N, w.H), w.beta)
    s0 = 0.02 * rng.standard_normal((N, w.H, w.dk, w.dv))
    return dict(q=_cast(q, w.dtype, device), k=_cast(k, w.dtype, device),
                v=_cast(v, w.dtype, device), beta=_cast(beta, w.dtype, device),
                s0=torch.from_numpy(s0).float().to(device))


def to_f64(t) -> np.ndarray | None:
    """Exact upcast of a (possibly bf16, possibly device) tensor to numpy float64."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def length_mix(n: int, total: int, seed: int) -> list:
    """n sequence lengths summing to `total`, with log-uniform shares over a
    64x range (a few long sequences and many short ones, as a packed training
    or serving batch holds them)."""
    rng = np.random.default_rng(seed)
    share = np.exp(rng.uniform(0.0, np.log(64.0), n))
    lengths = np.floor(share / share.sum() * total).astype(np.int64)
    lengths[np.argmax(lengths)] += total - int(lengths.sum())
    return [int(x) for x in lengths]


def generate_packed(w: Workload, lengths, device="cpu", H: int | None = None, seed: int | None = None,
                    lead: int = 0, tail: int = 0) -> dict:
    """Packed variable-length inputs with the distributions of workload w:
    sequences of the given lengths back to back, after `lead` and before
    `tail` tokens that belong to no sequence."""
    H = w.H if H is None else H
    N = len(lengths)
    T = lead + int(sum(lengths)) + tail
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = _qk(rng, (T, H, w.dk), w.qk, is_key=False)
    k = _qk(rng, (T, H, w.dk), w.qk, is_key=True)
    v = rng.standard_normal((T, H, w.dv))
    beta = _beta(rng, (T, H), w.beta)
    if w.spikes > 0:
        v[rng.random(T) < w.spikes] *= 100.0
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64) + lead
    s0 = None
    if w.s0 == "n002":
        s0 = torch.from_numpy(0.02 * rng.standard_normal((N, H, w.dk, w.dv))).float().to(device)
    return dict(q=_cast(q, w.dtype, device), k=_cast(k, w.dtype, device), v=_cast(v, w.dtype, device),
                beta=_cast(beta, w.dtype, device), s0=s0,
                cu_seqlens=torch.from_numpy(cu.astype(np.int32)).to(device))
