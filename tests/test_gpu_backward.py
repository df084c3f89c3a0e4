"""The chunked backward pass (efla_chunk_bwd) against the fp64 oracle's
reverse-mode gradients on the same inputs.  Error per gradient tensor is
normwise (max|x - y| / max|y|), with the forward pass's bounds: 1e-4 for fp32
inputs, 2e-2 for bf16 inputs (bf16 operands and gradients, fp32 accumulation).
bf16 inputs take the bf16 matrix-core chunk kernel where d_k and the chunk are
multiples of 32 and d_v of 32, else the fp32 one (EFLA_BWD_IMPL=fp32 forces it)."""
import numpy as np
import pytest
import torch

import oracle
from delta_rule_sequence_efla_amd import efla
from delta_rule_sequence_efla_amd import workloads as W
from delta_rule_sequence_efla_amd.workloads import to_f64
from tests._util import dtype_name, normwise, require_gpu

pytestmark = pytest.mark.gpu

GRAD_TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("dq", "dk", "dv", "dbeta", "ds0")


def _grads(inp, chunk, seed, rule="exact", with_dsf=True):
    q, k, v, beta, s0 = inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"]
    g = torch.Generator().manual_seed(seed)
    d_o = torch.randn(v.shape, generator=g).to(v.dtype).cuda()
    B, L, H, dk = k.shape
    dsf = torch.randn((B, H, dk, v.shape[-1]), generator=g).cuda() if with_dsf else None
    got = efla.efla_chunk_bwd(q, k, v, beta, d_o, s0, dsf, chunk=chunk, rule=rule)
    torch.cuda.synchronize()
    want = oracle.backward(to_f64(q), to_f64(k), to_f64(v), to_f64(beta), to_f64(s0), to_f64(d_o),
                           to_f64(dsf), rule=rule)
    return [to_f64(x) for x in got], want


def _check(inp, chunk, label, seed=0, rule="exact", with_dsf=True, tol=None):
    got, want = _grads(inp, chunk, seed, rule, with_dsf)
    tol = tol or GRAD_TOL[dtype_name(inp["q"])]
    errs = {n: normwise(a, b) for n, a, b in zip(NAMES, got, want)}
    print(f"[bwd] {label}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    for n, a in zip(NAMES, got):
        assert np.isfinite(a).all(), n
    bad = {n: e for n, e in errs.items() if e > tol}
    assert not bad, f"{label}: {bad} above {tol}"


SHAPES = [
    # dtype, dk, dv, chunk, L
    ("f32", 16, 16, 16, 64),
    ("f32", 32, 64, 32, 75),
    ("f32", 64, 32, 16, 33),
    ("f32", 128, 128, 64, 130),
    ("f32", 128, 16, 32, 47),
    ("bf16", 16, 32, 16, 50),
    ("bf16", 32, 32, 32, 33),
    ("bf16", 64, 64, 64, 300),
    ("bf16", 128, 128, 64, 257),
    ("bf16", 64, 128, 32, 129),
    ("bf16", 128, 16, 32, 47),    # d_v not a multiple of 32: the fp32 chunk kernel
]


@pytest.mark.parametrize("dt,dk,dv,chunk,L", SHAPES, ids=lambda x: str(x))
def test_backward_matches_oracle(dt, dk, dv, chunk, L):
    require_gpu()
    w, = (W.get("shape_340m", dtype=dt, dk=dk, dv=dv, chunk=chunk),)
    inp = W.generate(w, device="cuda", B=2, L=L, H=2, seed=900 + dk + dv + chunk + L)
    _check(inp, chunk, f"{dt} dk{dk} dv{dv} C{chunk} L{L}", seed=L)


@pytest.mark.parametrize("dk,dv,chunk,L,B,H", [(128, 64, 32, 97, 2, 4), (32, 128, 64, 200, 1, 8),
                                                (64, 32, 64, 65, 4, 4)], ids=lambda x: str(x))
def test_backward_bf16_grouped_state_pass(dk, dv, chunk, L, B, H):
    """bf16 matrix-core kernels with B*H a multiple of 8, where the state pass
    numbers its workgroups so that the value blocks of one (b, h) share an XCD,
    at d_k / chunk pairs the other cases leave out, with ragged last chunks."""
    require_gpu()
    w = W.get("shape_340m", dtype="bf16", dk=dk, dv=dv, chunk=chunk)
    inp = W.generate(w, device="cuda", B=B, L=L, H=H, seed=940 + dk + dv + chunk + L)
    _check(inp, chunk, f"bf16 dk{dk} dv{dv} C{chunk} L{L} B{B} H{H}", seed=L + 1)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_euler_rule(dt):
    require_gpu()
    w = W.get("shape_340m", dtype=dt, dk=64, dv=64, chunk=32)
    inp = W.generate(w, device="cuda", B=2, L=100, H=2, seed=931)
    _check(inp, 32, f"euler {dt}", seed=3, rule="euler")


def test_backward_unnormalised_and_stiff():
    require_gpu()
    # tiny_fp32's N(0,1) keys (lambda ~ 16) and the stiff workload's keys and beta (beta*lambda to ~1e4)
    w = W.get("tiny_fp32")
    _check(W.generate(w, device="cuda", seed=932), 16, "tiny_fp32", seed=4)
    ws = W.get("stiff_64k", dtype="f32", dk=32, dv=32, chunk=32)
    _check(W.generate(ws, device="cuda", B=1, L=200, H=2, seed=933), 32, "stiff fp32", seed=5)
    wb = W.get("stiff_64k", dk=64, dv=64)
    _check(W.generate(wb, device="cuda", B=1, L=300, H=2, seed=934), 64, "stiff bf16", seed=6)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_optional_state_gradients_and_empty_sequence(dt):
    require_gpu()
    w = W.get("shape_340m", dtype=dt, dk=32, dv=32, chunk=32)
    inp = W.generate(w, device="cuda", B=1, L=70, H=2, seed=935)
    _check(inp, 32, f"{dt}: no final-state gradient", seed=7, with_dsf=False)
    inp0 = W.generate(w, device="cuda", B=1, L=0, H=2, seed=936)
    dsf = torch.randn(1, 2, 32, 32, device="cuda")
    d_o = torch.empty(1, 0, 2, 32, device="cuda", dtype=inp0["q"].dtype)
    dq, dk, dv, db, ds0 = efla.efla_chunk_bwd(inp0["q"], inp0["k"], inp0["v"], inp0["beta"], d_o, inp0["s0"], dsf,
                                              chunk=32)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.equal(ds0, dsf)
    # without ds0 the other gradients are the same bits
    g = torch.Generator().manual_seed(8)
    d_o = torch.randn(inp["v"].shape, generator=g).to(inp["v"].dtype).cuda()
    args = (inp["q"], inp["k"], inp["v"], inp["beta"], d_o, inp["s0"], None)
    full = efla.efla_chunk_bwd(*args, chunk=32)
    part = efla.efla_chunk_bwd(*args, chunk=32, want_ds0=False)
    torch.cuda.synchronize()
    assert part[4] is None and all(torch.equal(a, b) for a, b in zip(full[:4], part[:4]))


def test_backward_1p3b_heads_short_sequence():
    """The 1.3B head configuration (d = 128, chunk 64, bf16) on a short sequence."""
    require_gpu()
    w = W.get("shape_1p3b")
    inp = W.generate(w, device="cuda", B=1, L=512, H=4, seed=937)
    _check(inp, 64, "shape_1p3b heads, L=512", seed=8)


@pytest.mark.slow
def test_backward_full_1p3b_shape():
    """The benchmark workload (B=4, H=16, L=4096, d=128, chunk 64, bf16) in the
    launch configuration bench.py times."""
    require_gpu()
    w = W.get("shape_1p3b")
    _check(W.generate(w, device="cuda"), 64, "shape_1p3b full", seed=9)


@pytest.mark.parametrize("impl,ut", [("fp32", "workgroup"), ("fp32", "wave"), ("bf16", "wave"),
                                     ("bf16", "workgroup")])
def test_backward_bf16_inputs_both_chunk_kernels(impl, ut, monkeypatch):
    """bf16 inputs through the fp32 chunk and state kernels (P in fp32) with
    either UT transform, and through the bf16 kernels (P in bf16, so the
    one-wavefront-per-chunk UT transform runs even where the workgroup one is
    asked for), at the 1.3B head configuration with a ragged last chunk and the
    Euler rule too."""
    require_gpu()
    if impl == "fp32":
        monkeypatch.setenv("EFLA_BWD_IMPL", "fp32")
    else:
        monkeypatch.delenv("EFLA_BWD_IMPL", raising=False)
    if ut == "workgroup":
        monkeypatch.setenv("EFLA_UT_IMPL", "workgroup")
    else:
        monkeypatch.delenv("EFLA_UT_IMPL", raising=False)
    w = W.get("shape_1p3b")
    inp = W.generate(w, device="cuda", B=1, H=3, L=200, seed=930)
    _check(inp, 64, f"bf16 inputs, {impl} chunk kernel, {ut} UT", seed=31)
    _check(inp, 64, f"bf16 inputs, {impl} chunk kernel, {ut} UT, Euler rule", seed=32, rule="euler")


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64)])
def test_backward_chunk_state_kernels_agree(dk, dv, monkeypatch):
    """The chunk-start states from the state-only kernel (stored transposed)
    and from the role kernel (EFLA_BWD_STATES=roles, stored row-major) give the
    same gradients up to the order of fp32 sums, with a ragged last chunk and
    an initial state."""
    require_gpu()
    w = W.get("shape_340m", dk=dk, dv=dv, chunk=64)
    inp = W.generate(w, device="cuda", B=2, H=3, L=300, seed=940 + dk + dv)
    g = torch.Generator().manual_seed(41)
    d_o = torch.randn(inp["v"].shape, generator=g).to(inp["v"].dtype).cuda()
    dsf = torch.randn((2, 3, dk, dv), generator=g).cuda()
    args = (inp["q"], inp["k"], inp["v"], inp["beta"], d_o, inp["s0"], dsf)
    monkeypatch.delenv("EFLA_BWD_STATES", raising=False)
    a = efla.efla_chunk_bwd(*args, chunk=64)
    monkeypatch.setenv("EFLA_BWD_STATES", "roles")
    b = efla.efla_chunk_bwd(*args, chunk=64)
    torch.cuda.synchronize()
    errs = {n: normwise(to_f64(x), to_f64(y)) for n, x, y in zip(NAMES, a, b)}
    print(f"[bwd] state kernels dk{dk} dv{dv}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    assert all(e <= 5e-3 for e in errs.values()), errs


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64)])
@pytest.mark.parametrize("impl", ["state-only", "stager"])
def test_backward_both_reverse_passes(dk, dv, impl, monkeypatch):
    """Both reverse passes over the chunks against the oracle: the one in the
    state-only form (through Q - P T K, dS stored transposed; the default) and
    the sixteen-wavefront kernel (EFLA_BWD_REVERSE=stager, through P^T dO),
    with a ragged last chunk, an initial state and a final-state gradient."""
    require_gpu()
    if impl == "stager":
        monkeypatch.setenv("EFLA_BWD_REVERSE", "stager")
    else:
        monkeypatch.delenv("EFLA_BWD_REVERSE", raising=False)
    w = W.get("shape_340m", dk=dk, dv=dv, chunk=64)
    inp = W.generate(w, device="cuda", B=2, H=3, L=300, seed=970 + dk + dv)
    _check(inp, 64, f"{impl} reverse pass dk{dk} dv{dv}", seed=43)
    _check(inp, 64, f"{impl} reverse pass dk{dk} dv{dv}, Euler rule", seed=44, rule="euler")
