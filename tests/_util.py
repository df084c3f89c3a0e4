"""Shared helpers for the parity tests: the error metric and oracle calls.

Error metric (the reading of "max relative error" used throughout): normwise
per tensor, max|x - y| / max|y|, with y the fp64 oracle.
"""
import numpy as np
import torch

import oracle
from delta_rule_sequence_efla_amd.workloads import to_f64

TOL = {
    "f32": {"o": 1e-4, "s": 1e-4},
    "bf16": {"o": 2e-2, "s": 1e-2},
}


def normwise(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    denom = np.abs(ref).max() if ref.size else 0.0
    if denom == 0.0:
        return float(np.abs(x - ref).max()) if ref.size else 0.0
    return float(np.abs(x - ref).max() / denom)


def dtype_name(t: torch.Tensor) -> str:
    return {torch.float32: "f32", torch.bfloat16: "bf16"}[t.dtype]


def oracle_forward(inp: dict, nthreads=None, rule="exact"):
    """fp64 oracle on the exact values handed to the GPU."""
    return oracle.forward(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]),
                          to_f64(inp["beta"]), to_f64(inp.get("s0")), nthreads=nthreads, rule=rule)


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
