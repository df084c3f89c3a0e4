"""Packed variable-length batches through efla_chunk_fwd_varlen, against the
fp64 oracle run sequence by sequence (tolerances as in test_gpu_parity)."""
import numpy as np
import pytest
import torch

import oracle
from delta_rule_sequence_efla_amd import efla
from delta_rule_sequence_efla_amd import workloads as W
from delta_rule_sequence_efla_amd.workloads import to_f64
from tests._util import TOL, dtype_name, normwise, require_gpu

pytestmark = pytest.mark.gpu

# lengths around every chunk boundary, empty sequences, one long sequence
MIX = [0, 1, 15, 16, 17, 63, 64, 65, 0, 200, 31, 130, 7, 1]


def _check(inp, chunk, label, rule="exact", lead=0, tail=0):
    q, k, v, beta, cu, s0 = inp["q"], inp["k"], inp["v"], inp["beta"], inp["cu_seqlens"], inp["s0"]
    sentinel = torch.full(v.shape, 7.0, dtype=v.dtype, device=v.device)
    o, sf = efla.efla_chunk_fwd_varlen(q, k, v, beta, cu, s0, chunk=chunk, o=sentinel, rule=rule)
    torch.cuda.synchronize()
    ro, rs = oracle.forward_varlen(to_f64(q), to_f64(k), to_f64(v), to_f64(beta), cu.cpu().numpy(),
                                   to_f64(s0), rule=rule)
    cuh = cu.cpu().numpy()
    a, e = int(cuh[0]), int(cuh[-1])
    og = to_f64(o)
    tol = TOL[dtype_name(q)]
    eo, es = normwise(og[a:e], ro[a:e]), normwise(to_f64(sf), rs)
    print(f"[varlen] {label}: o err {eo:.3e}, S err {es:.3e}", flush=True)
    assert np.isfinite(og[a:e]).all() and np.isfinite(to_f64(sf)).all()
    assert eo <= tol["o"] and es <= tol["s"]
    assert (og[:a] == 7.0).all() and (og[e:] == 7.0).all()   # outside every sequence: untouched
    return o, sf


CASES = [
    # dtype, dk, dv, chunk, implementation
    ("f32", 64, 32, 32, None),
    ("f32", 16, 16, 16, None),
    ("bf16", 128, 128, 64, "split"),
    ("bf16", 64, 64, 64, "split"),
    ("bf16", 128, 128, 64, "roles"),
    ("bf16", 128, 128, 64, "generic"),
    ("bf16", 64, 128, 32, "roles"),
    ("bf16", 32, 64, 64, "tile"),       # the tile kernel takes dense batches: falls back to roles
    ("bf16", 16, 32, 16, None),         # generic kernels (d_k 16, chunk 16)
    ("bf16", 128, 16, 32, "roles"),     # one 16-column value block
]


@pytest.mark.parametrize("ut", ["wave", "workgroup"])
@pytest.mark.parametrize("dt,dk,dv,chunk,impl", CASES, ids=lambda x: str(x))
def test_varlen_matches_oracle(dt, dk, dv, chunk, impl, ut, monkeypatch):
    require_gpu()
    if impl:
        monkeypatch.setenv("EFLA_RECURRENCE_IMPL", impl)
    monkeypatch.setenv("EFLA_UT_IMPL", ut)
    w = W.get("shape_340m", dtype=dt, dk=dk, dv=dv, chunk=chunk)
    inp = W.generate_packed(w, MIX, device="cuda", H=3, seed=800 + dk + dv + chunk, lead=5, tail=9)
    _check(inp, chunk, f"{dt} dk{dk} dv{dv} C{chunk} {impl} ut {ut}", lead=5, tail=9)


def test_varlen_equal_lengths_is_bitwise_the_dense_call():
    require_gpu()
    w, B, L = W.get("shape_1p3b"), 3, 300
    inp = W.generate(w, device="cuda", B=B, L=L, H=4, seed=811)
    o, sf = efla.efla_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"], chunk=64)
    cu = torch.arange(B + 1, dtype=torch.int32, device="cuda") * L
    ov, sv = efla.efla_chunk_fwd_varlen(inp["q"].view(B * L, 4, -1), inp["k"].view(B * L, 4, -1),
                                        inp["v"].view(B * L, 4, -1), inp["beta"].view(B * L, 4), cu,
                                        inp["s0"], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(ov.view_as(o), o) and torch.equal(sv, sf)


def test_varlen_1p3b_mix_and_euler():
    require_gpu()
    w = W.get("varlen_1p3b")
    inp = W.generate_packed(w, W.length_mix(w.B, 2048, seed=812), device="cuda", H=4, seed=813)
    _check(inp, 64, "varlen_1p3b-shaped mix (4 heads, 2048 tokens)")
    _check(inp, 64, "same, Euler rule", rule="euler")


def test_varlen_empty_batches():
    require_gpu()
    w = W.get("shape_340m", dk=32, dv=32, chunk=32)
    inp = W.generate_packed(w, [0, 0, 0], device="cuda", H=2, seed=814)
    o, sf = efla.efla_chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["beta"], inp["cu_seqlens"],
                                       inp["s0"], chunk=32)
    torch.cuda.synchronize()
    assert torch.equal(sf, inp["s0"])
    _, sf0 = efla.efla_chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["beta"], inp["cu_seqlens"],
                                        None, chunk=32)
    torch.cuda.synchronize()
    assert torch.count_nonzero(sf0) == 0


def _schedule(ws, N, H, T, dk, dv, chunk, dtype):
    """The rank -> sequence schedule the call left in its workspace: int32 per
    sequence after the 256-byte-aligned T slots."""
    esz = torch.empty((), dtype=dtype).element_size()
    off = (H * (T // chunk + N) * chunk * chunk * esz + 255) // 256 * 256
    return ws[off:off + 4 * N].view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("lengths", [MIX, "mix"], ids=["boundary_mix", "1p3b_mix"])
def test_varlen_schedule_is_longest_first(lengths):
    """Sequences are handed to the recurrence by chunk count, longest first,
    ties by index: the schedule is a permutation with non-increasing counts."""
    require_gpu()
    w = W.get("varlen_1p3b")
    if lengths == "mix":
        lengths = W.length_mix(w.B, 2048, seed=815)
    inp = W.generate_packed(w, lengths, device="cuda", H=2, seed=816, lead=3, tail=4)
    q, cu = inp["q"], inp["cu_seqlens"]
    N, T, H = cu.numel() - 1, q.shape[0], q.shape[1]
    n = efla.efla_chunk_fwd_varlen_workspace_size(N, H, T, w.dk, w.dv, w.chunk, q.dtype)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    _check(dict(inp), w.chunk, f"schedule check, {N} sequences", lead=3, tail=4)
    efla.efla_chunk_fwd_varlen(q, inp["k"], inp["v"], inp["beta"], cu, inp["s0"], chunk=w.chunk, workspace=ws)
    torch.cuda.synchronize()
    order = _schedule(ws, N, H, T, w.dk, w.dv, w.chunk, q.dtype)
    assert sorted(order.tolist()) == list(range(N))
    cuh = cu.cpu().numpy().astype(np.int64)
    nc = (cuh[1:] - cuh[:-1] + w.chunk - 1) // w.chunk
    keys = [(-int(nc[u]), int(u)) for u in order]
    assert keys == sorted(keys)


def test_varlen_many_sequences_unordered_path():
    """Beyond the ordered-schedule limit (4096 sequences) the recurrence takes
    sequences in index order; results still match the oracle."""
    require_gpu()
    w = W.get("shape_340m", dk=16, dv=16, chunk=16)
    rng = np.random.default_rng(817)
    lengths = rng.integers(0, 5, size=4100).tolist()
    lengths[17] = 40   # one sequence of several chunks
    inp = W.generate_packed(w, lengths, device="cuda", H=1, seed=818)
    _check(inp, 16, "4100 short sequences")


@pytest.mark.slow
def test_varlen_1p3b_full_size():
    """The packed workload the benchmark times, at full size: 16 sequences of a
    seeded log-uniform length mix, 16384 tokens, 16 heads of d = 128."""
    require_gpu()
    w = W.get("varlen_1p3b")
    inp = W.generate_packed(w, W.length_mix(w.B, w.L, seed=w.seed), device="cuda")
    _check(inp, w.chunk, "varlen_1p3b full size")
