"""efla_chunk_fwd_segmented (the intra-GPU segment scan) against the fp64
oracle, and against the plain chunked forward, with the forward pass's
tolerances."""
import numpy as np
import pytest
import torch

from delta_rule_sequence_efla_amd import efla
from delta_rule_sequence_efla_amd import workloads as W
from delta_rule_sequence_efla_amd.workloads import to_f64
from tests._util import TOL, dtype_name, normwise, oracle_forward, require_gpu

pytestmark = pytest.mark.gpu


def _check(inp, chunk, segments, label, rule="exact"):
    o, sf = efla.efla_chunk_fwd_segmented(inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"], chunk=chunk,
                                          segments=segments, rule=rule)
    torch.cuda.synchronize()
    ro, rs = oracle_forward(inp, rule=rule)
    tol = TOL[dtype_name(inp["q"])]
    eo, es = normwise(to_f64(o), ro), normwise(to_f64(sf), rs)
    print(f"[seg] {label}: o err {eo:.3e}, S err {es:.3e}", flush=True)
    assert np.isfinite(to_f64(o)).all() and np.isfinite(to_f64(sf)).all()
    assert eo <= tol["o"] and es <= tol["s"], label
    return o, sf


CASES = [
    # dtype, dk, dv, chunk, L, segments
    ("f32", 16, 16, 16, 200, 4),
    ("f32", 64, 32, 32, 300, 3),        # segments not dividing the chunk count, ragged tail
    ("f32", 128, 128, 64, 257, 5),      # more segments than chunks' worth: clamped
    ("bf16", 128, 128, 64, 1000, 4),    # state-only pass for N and M, split kernel for the output
    ("bf16", 64, 64, 64, 700, 3),       # state-only pass at d_k = 64
    ("bf16", 128, 64, 64, 900, 5),      # d_v < d_k: the last column blocks write M only
    ("bf16", 64, 128, 64, 450, 2),      # d_v > d_k: the last column blocks write N only
    ("bf16", 64, 128, 32, 513, 7),
    ("bf16", 16, 32, 16, 300, 3),       # generic kernels
    ("bf16", 32, 32, 64, 640, 10),      # one chunk per segment
    ("bf16", 128, 16, 32, 200, 2),      # 16-column value blocks; transition has 128 columns
]


@pytest.mark.parametrize("dt,dk,dv,chunk,L,segments", CASES, ids=lambda x: str(x))
def test_segmented_matches_oracle(dt, dk, dv, chunk, L, segments):
    require_gpu()
    w = W.get("shape_340m", dtype=dt, dk=dk, dv=dv, chunk=chunk)
    inp = W.generate(w, device="cuda", B=2, L=L, H=2, seed=950 + dk + dv + L + segments)
    _check(inp, chunk, segments, f"{dt} dk{dk} dv{dv} C{chunk} L{L} G{segments}")


def test_segmented_stiff_and_euler():
    require_gpu()
    ws = W.get("stiff_64k")
    inp = W.generate(ws, device="cuda", B=1, L=4096, H=4, seed=961)
    o, sf = _check(inp, 64, 8, "stiff, 4096 tokens, 8 segments")
    o1, s1 = efla.efla_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"], chunk=64)
    torch.cuda.synchronize()
    assert normwise(to_f64(o), to_f64(o1)) <= 2e-2 and normwise(to_f64(sf), to_f64(s1)) <= 1e-2
    w = W.get("shape_340m", dk=64, dv=64, chunk=32)
    _check(W.generate(w, device="cuda", B=1, L=700, H=2, seed=962), 32, 6, "euler", rule="euler")


@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64), (64, 128)])
def test_state_only_pass_matches_two_passes(dk, dv, monkeypatch):
    """N and M from the one state-only pass against the two passes of the
    general recurrence (EFLA_SEG_STATES=0); both round S to bf16 for the
    products, so they agree to well inside the forward tolerances."""
    require_gpu()
    w = W.get("shape_340m", dk=dk, dv=dv, chunk=64)
    inp = W.generate(w, device="cuda", B=2, L=1300, H=3, seed=964 + dk + dv)
    args = (inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"])
    o1, s1 = efla.efla_chunk_fwd_segmented(*args, chunk=64, segments=5)
    monkeypatch.setenv("EFLA_SEG_STATES", "0")
    o2, s2 = efla.efla_chunk_fwd_segmented(*args, chunk=64, segments=5)
    torch.cuda.synchronize()
    eo, es = normwise(to_f64(o1), to_f64(o2)), normwise(to_f64(s1), to_f64(s2))
    print(f"[seg] state-only vs two passes dk{dk} dv{dv}: o {eo:.3e}, S {es:.3e}", flush=True)
    assert eo <= 5e-3 and es <= 5e-3


def test_one_segment_is_the_plain_pass():
    require_gpu()
    w = W.get("shape_340m", dtype="f32", dk=32, dv=32, chunk=32)
    inp = W.generate(w, device="cuda", B=2, L=150, H=2, seed=963)
    o, sf = efla.efla_chunk_fwd_segmented(inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"], chunk=32, segments=1)
    o1, s1 = efla.efla_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"], chunk=32)
    torch.cuda.synchronize()
    # one segment: the incoming state is s0 and the output pass is the plain recurrence on the packed view
    assert normwise(to_f64(o), to_f64(o1)) <= 1e-6 and normwise(to_f64(sf), to_f64(s1)) <= 1e-5


@pytest.mark.slow
def test_segmented_full_stiff_64k():
    """The stiff long-context workload (B=1, H=16, L=65536) in the launch
    configuration bench.py times."""
    require_gpu()
    w = W.get("stiff_64k")
    inp = W.generate(w, device="cuda")
    _check(inp, 64, efla.default_segments(w.B, w.H, w.L, w.dv, w.chunk), "stiff_64k full")
