"""The training pair (efla_chunk_fwd_train, efla_chunk_bwd_train): the forward
pass stores every chunk's UT-transform quantities and start state in the
backward workspace and the backward pass reads them instead of running the UT
transform and the recurrence again.

Checked here: the forward's outputs are bitwise those of efla_chunk_fwd; each
stored state equals the oracle's state after that chunk's prefix of tokens
(the definition of a chunk-start state) within bf16 rounding; the gradients
match the oracle's reverse-mode ones (the backward tolerance, 2e-2 normwise
for bf16) and are bitwise efla_chunk_bwd's (the stored states are the bits the
backward's state-only pass computes: the same products in the same order);
shapes without stored states give exactly
efla_chunk_fwd / efla_chunk_bwd; a second forward pass into the same
workspace leaves nothing of the first."""
import numpy as np
import pytest
import torch

import oracle
from delta_rule_sequence_efla_amd import efla
from delta_rule_sequence_efla_amd import workloads as W
from delta_rule_sequence_efla_amd.workloads import to_f64
from tests._util import normwise, require_gpu

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "ds0")
GRAD_TOL = 2e-2
STATE_TOL = 1e-2     # bf16 operand values of a state (2^-9 relative rounding) after fp32 accumulation

# d_k, d_v, L (ragged last chunk where L % 64 != 0), B, H
SHAPES = [(128, 128, 300, 2, 3), (64, 64, 257, 2, 2), (128, 64, 130, 1, 4), (64, 128, 64, 2, 2),
          (128, 32, 190, 3, 1), (64, 32, 70, 1, 1)]   # one value block; a single sequence and head


def _al(x):
    return (x + 255) // 256 * 256


def _stored_states(ws, B, H, L, dk, dv, C=64):
    """The workspace's state region as [B, H, NC, dk, dv] float64 (stored
    [slots][dv][dk] in bf16, slot (b H + h) NC + n; after T (bf16), X, P
    (fp32) and the coefficients, each region 256-byte aligned)."""
    nc = (L + C - 1) // C
    slots = B * H * nc
    off = _al(slots * C * C * 2) + 2 * _al(slots * C * C * 4) + _al(slots * C * 4)
    n = slots * dk * dv
    raw = ws[off:off + 2 * n].view(torch.bfloat16).reshape(B, H, nc, dv, dk)
    return to_f64(raw.transpose(-1, -2))


def _inputs(dk, dv, L, B, H, seed):
    w = W.get("shape_340m", dk=dk, dv=dv, chunk=64)
    return W.generate(w, device="cuda", B=B, L=L, H=H, seed=seed)


def _cotangents(inp, seed):
    g = torch.Generator().manual_seed(seed)
    B, L, H, dk = inp["k"].shape
    dv = inp["v"].shape[-1]
    d_o = torch.randn(inp["v"].shape, generator=g).to(inp["v"].dtype).cuda()
    dsf = torch.randn((B, H, dk, dv), generator=g).cuda()
    return d_o, dsf


@pytest.mark.parametrize("rule", ["exact", "euler"])
@pytest.mark.parametrize("dk,dv,L,B,H", SHAPES, ids=lambda x: str(x))
def test_train_forward_is_the_forward(dk, dv, L, B, H, rule):
    require_gpu()
    assert efla.efla_chunk_train_saves_states(dk, dv, 64, torch.bfloat16)
    inp = _inputs(dk, dv, L, B, H, 1200 + dk + dv + L)
    args = (inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"])
    o, sf = efla.efla_chunk_fwd(*args, chunk=64, rule=rule)
    o2, sf2, _ = efla.efla_chunk_fwd_train(*args, chunk=64, rule=rule)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(sf, sf2)


@pytest.mark.parametrize("dk,dv,L,B,H", SHAPES, ids=lambda x: str(x))
def test_train_stored_states_are_prefix_states(dk, dv, L, B, H):
    """State n stored by the forward pass = the oracle's final state over the
    first 64 n tokens (from s0), for every chunk of every sequence."""
    require_gpu()
    inp = _inputs(dk, dv, L, B, H, 1300 + dk + dv + L)
    _, _, ws = efla.efla_chunk_fwd_train(inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"], chunk=64)
    torch.cuda.synchronize()
    got = _stored_states(ws.cpu(), B, H, L, dk, dv)
    q, k, v, beta, s0 = (to_f64(inp[n]) for n in ("q", "k", "v", "beta", "s0"))
    worst = 0.0
    for n in range(got.shape[2]):
        t = 64 * n
        want = s0 if t == 0 else oracle.forward(q[:, :t], k[:, :t], v[:, :t], beta[:, :t], s0)[1]
        for b in range(B):
            for h in range(H):
                worst = max(worst, normwise(got[b, h, n], want[b, h]))
    print(f"[train] stored states dk{dk} dv{dv} L{L}: worst {worst:.2e}", flush=True)
    assert worst <= STATE_TOL


@pytest.mark.parametrize("rule", ["exact", "euler"])
@pytest.mark.parametrize("dk,dv,L,B,H", SHAPES, ids=lambda x: str(x))
def test_train_backward_matches_oracle_and_bwd(dk, dv, L, B, H, rule):
    require_gpu()
    inp = _inputs(dk, dv, L, B, H, 1400 + dk + dv + L)
    d_o, dsf = _cotangents(inp, L + dk)
    q, k, v, beta, s0 = inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"]
    _, _, ws = efla.efla_chunk_fwd_train(q, k, v, beta, s0, chunk=64, rule=rule)
    got = efla.efla_chunk_bwd_train(q, k, v, beta, d_o, ws, s0, dsf, chunk=64, rule=rule)
    ref = efla.efla_chunk_bwd(q, k, v, beta, d_o, s0, dsf, chunk=64, rule=rule)
    torch.cuda.synchronize()
    want = oracle.backward(to_f64(q), to_f64(k), to_f64(v), to_f64(beta), to_f64(s0), to_f64(d_o), to_f64(dsf),
                           rule=rule)
    errs = {n: normwise(to_f64(a), b) for n, a, b in zip(NAMES, got, want)}
    print(f"[train] bwd dk{dk} dv{dv} L{L} {rule}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()),
          flush=True)
    for n, a in zip(NAMES, got):
        assert np.isfinite(to_f64(a)).all(), n
    assert all(e <= GRAD_TOL for e in errs.values()), errs
    assert all(torch.equal(a, b) for a, b in zip(got, ref)), "gradients differ from efla_chunk_bwd's"



def test_train_workspace_reuse_and_backward_without_state_gradients():
    """A second forward pass (new inputs, same workspace) replaces every stored
    state: the backward pass then gives the new inputs' gradients; without
    ds_final and ds0 as well."""
    require_gpu()
    a = _inputs(128, 128, 200, 2, 2, 1501)
    b = _inputs(128, 128, 200, 2, 2, 1502)
    _, _, ws = efla.efla_chunk_fwd_train(a["q"], a["k"], a["v"], a["beta"], a["s0"], chunk=64)
    efla.efla_chunk_fwd_train(b["q"], b["k"], b["v"], b["beta"], None, chunk=64, workspace=ws)
    d_o, _ = _cotangents(b, 7)
    got = efla.efla_chunk_bwd_train(b["q"], b["k"], b["v"], b["beta"], d_o, ws, None, None, chunk=64,
                                    want_ds0=False)
    torch.cuda.synchronize()
    assert got[4] is None
    want = oracle.backward(to_f64(b["q"]), to_f64(b["k"]), to_f64(b["v"]), to_f64(b["beta"]), None, to_f64(d_o),
                           None)
    errs = {n: normwise(to_f64(x), y) for n, x, y in zip(NAMES[:4], got[:4], want[:4])}
    print("[train] reused workspace: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    assert all(e <= GRAD_TOL for e in errs.values()), errs


@pytest.mark.parametrize("dt,dk,dv,chunk,L", [("f32", 32, 64, 32, 75), ("bf16", 128, 128, 32, 97),
                                              ("bf16", 128, 16, 64, 70), ("bf16", 32, 32, 64, 100)],
                         ids=lambda x: str(x))
def test_train_pair_without_stored_states_is_fwd_then_bwd(dt, dk, dv, chunk, L):
    require_gpu()
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    assert not efla.efla_chunk_train_saves_states(dk, dv, chunk, tdt)
    w = W.get("shape_340m", dtype=dt, dk=dk, dv=dv, chunk=chunk)
    inp = W.generate(w, device="cuda", B=2, L=L, H=2, seed=1600 + dk + dv + chunk)
    d_o, dsf = _cotangents(inp, 11)
    q, k, v, beta, s0 = inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"]
    o, sf = efla.efla_chunk_fwd(q, k, v, beta, s0, chunk=chunk)
    o2, sf2, ws = efla.efla_chunk_fwd_train(q, k, v, beta, s0, chunk=chunk)
    got = efla.efla_chunk_bwd_train(q, k, v, beta, d_o, ws, s0, dsf, chunk=chunk)
    ref = efla.efla_chunk_bwd(q, k, v, beta, d_o, s0, dsf, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(sf, sf2)
    assert all(torch.equal(x, y) for x, y in zip(got, ref))


def test_train_pair_empty_sequence():
    require_gpu()
    inp = _inputs(128, 128, 0, 1, 2, 1700)
    s0 = inp["s0"]
    o, sf, ws = efla.efla_chunk_fwd_train(inp["q"], inp["k"], inp["v"], inp["beta"], s0, chunk=64)
    dsf = torch.randn(1, 2, 128, 128, device="cuda")
    d_o = torch.empty(1, 0, 2, 128, device="cuda", dtype=inp["q"].dtype)
    dq, dk, dv, db, ds0 = efla.efla_chunk_bwd_train(inp["q"], inp["k"], inp["v"], inp["beta"], d_o, ws, s0, dsf,
                                                    chunk=64)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(sf, s0) and dq.numel() == 0 and torch.equal(ds0, dsf)


@pytest.mark.slow
@pytest.mark.parametrize("rule", ["exact", "euler"])
def test_train_pair_full_1p3b_shape(rule):
    """The benchmark workload (B=4, H=16, L=4096, d=128, chunk 64, bf16) in the
    launch configuration the training step is timed in, under both rules:
    outputs bitwise those of efla_chunk_fwd, gradients bitwise those of
    efla_chunk_bwd (itself checked against the oracle at this size) and
    against the oracle's on sampled (b, h) pairs."""
    require_gpu()
    w = W.get("shape_1p3b")
    inp = W.generate(w, device="cuda")
    d_o, dsf = _cotangents(inp, 21)
    q, k, v, beta, s0 = inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"]
    o, sf = efla.efla_chunk_fwd(q, k, v, beta, s0, chunk=64, rule=rule)
    o2, sf2, ws = efla.efla_chunk_fwd_train(q, k, v, beta, s0, chunk=64, rule=rule)
    got = efla.efla_chunk_bwd_train(q, k, v, beta, d_o, ws, s0, dsf, chunk=64, rule=rule)
    ref = efla.efla_chunk_bwd(q, k, v, beta, d_o, s0, dsf, chunk=64, rule=rule)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(sf, sf2)
    assert all(torch.equal(a, b) for a, b in zip(got, ref)), "gradients differ from efla_chunk_bwd's"
    # (b, h) pairs run independently: the oracle on two of them
    for b, h in ((0, 0), (3, 11)):
        sl = lambda t: to_f64(t[b:b + 1, :, h:h + 1])
        want = oracle.backward(sl(q), sl(k), sl(v), sl(beta), to_f64(s0[b:b + 1, h:h + 1]), sl(d_o),
                               to_f64(dsf[b:b + 1, h:h + 1]), rule=rule)
        mine = [sl(got[0]), sl(got[1]), sl(got[2]), to_f64(got[3][b:b + 1, :, h:h + 1]),
                to_f64(got[4][b:b + 1, h:h + 1])]
        errs = {n: normwise(x, y) for n, x, y in zip(NAMES, mine, want)}
        print(f"[train] full shape (b{b}, h{h}) vs oracle: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()),
              flush=True)
        assert all(e <= GRAD_TOL for e in errs.values()), errs


@pytest.mark.parametrize("env", [("EFLA_BWD_CHUNK", "stager"), ("EFLA_BWD_REVERSE", "stager"),
                                 ("EFLA_BWD_IMPL", "fp32"), ("EFLA_BWD_STATES", "roles")],
                         ids=lambda e: f"{e[0]}={e[1]}")
def test_train_backward_under_every_kernel_choice(env, monkeypatch):
    """The paired backward with each backward kernel the environment can
    select (after a forward under the defaults): the stored states are read by
    the one-workgroup per-chunk kernel and by the sixteen-wavefront reverse
    pass too; with the fp32 kernels (and the state kernel choice, which the
    stored states make moot) everything is recomputed."""
    require_gpu()
    inp = _inputs(128, 128, 200, 2, 2, 1800)
    d_o, dsf = _cotangents(inp, 19)
    q, k, v, beta, s0 = inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"]
    for name in ("EFLA_BWD_CHUNK", "EFLA_BWD_REVERSE", "EFLA_BWD_IMPL", "EFLA_BWD_STATES"):
        monkeypatch.delenv(name, raising=False)
    _, _, ws = efla.efla_chunk_fwd_train(q, k, v, beta, s0, chunk=64)
    monkeypatch.setenv(*env)
    got = efla.efla_chunk_bwd_train(q, k, v, beta, d_o, ws, s0, dsf, chunk=64)
    torch.cuda.synchronize()
    want = oracle.backward(to_f64(q), to_f64(k), to_f64(v), to_f64(beta), to_f64(s0), to_f64(d_o), to_f64(dsf))
    errs = {n: normwise(to_f64(a), b) for n, a, b in zip(NAMES, got, want)}
    print(f"[train] {env[0]}={env[1]}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    assert all(e <= GRAD_TOL for e in errs.values()), errs
