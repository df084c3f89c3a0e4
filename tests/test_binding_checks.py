"""The Python binding rejects tensors whose shape, dtype or device does not
match what the kernels index, before anything reaches the C ABI (CPU only).

The library sees raw pointers, so a mismatched output or state would become
out-of-bounds device accesses; these tests replace the device check with one
that accepts host tensors and the library with a stub that fails the test if
any entry point is reached."""
import pytest
import torch

from delta_rule_sequence_efla_amd import efla


class _NoLaunch:
    def __getattr__(self, name):
        if name.endswith("_workspace_size"):
            return lambda *a: 1 << 20
        raise AssertionError(f"{name} reached the C ABI despite bad arguments")


@pytest.fixture
def host(monkeypatch):
    def dev(*ts, dtype=None):
        d = None
        for t in ts:
            if t is None:
                continue
            if dtype is not None and t.dtype != dtype:
                raise ValueError(f"expected dtype {dtype}, got {t.dtype}")
            if d is None:
                d = t.device
            elif t.device != d:
                raise ValueError("EFLA tensors must share one device")
        return d
    monkeypatch.setattr(efla, "_dev", dev)
    monkeypatch.setattr(efla, "lib", lambda: _NoLaunch())


def _inputs(B=2, L=8, H=3, dk=16, dv=32, dtype=torch.bfloat16):
    q = torch.zeros(B, L, H, dk, dtype=dtype)
    return q, q.clone(), torch.zeros(B, L, H, dv, dtype=dtype), torch.zeros(B, L, H, dtype=dtype)


BAD_FWD = [
    ("o", lambda B, L, H, dk, dv: {"o": torch.zeros(B, L, H, dv + 16, dtype=torch.bfloat16)}),
    ("o", lambda B, L, H, dk, dv: {"o": torch.zeros(B, L, H, dv, dtype=torch.float32)}),
    ("s_final", lambda B, L, H, dk, dv: {"s_final": torch.zeros(B, H, dk, dv + 1)}),
    ("s_final", lambda B, L, H, dk, dv: {"s_final": torch.zeros(B, H, dk, dv, dtype=torch.float64)}),
    ("s0", lambda B, L, H, dk, dv: {"s0": torch.zeros(B, H, dv, dk)}),
]


@pytest.mark.parametrize("what,extra", BAD_FWD)
def test_chunk_fwd_rejects_bad_outputs(host, what, extra):
    q, k, v, beta = _inputs()
    kw = extra(2, 8, 3, 16, 32)
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd(q, k, v, beta, kw.pop("s0", None), chunk=16, **kw)


def test_chunk_fwd_rejects_bad_inputs(host):
    q, k, v, beta = _inputs()
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd(q[:, :4], k, v, beta, chunk=16)
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd(q, k, v[:, :4], beta, chunk=16)
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd(q, k, v, beta[..., :1], chunk=16)
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd(q, k, v, beta.float(), chunk=16)


def test_recurrence_checks_every_tensor(host):
    q, k, v, beta = _inputs()
    ws = torch.zeros(1 << 10, dtype=torch.uint8)
    with pytest.raises(ValueError):   # q and k differ
        efla.efla_chunk_recurrence(q[:, :, :2], k, v, ws, chunk=16)
    with pytest.raises(ValueError):   # v has the wrong length
        efla.efla_chunk_recurrence(q, k, v[:, :4], ws, chunk=16)
    with pytest.raises(ValueError):   # s0 transposed
        efla.efla_chunk_recurrence(q, k, v, ws, s0=torch.zeros(2, 3, 32, 16), chunk=16)
    with pytest.raises(ValueError):   # o with the wrong value width
        efla.efla_chunk_recurrence(q, k, v, ws, o=torch.zeros(2, 8, 3, 16, dtype=torch.bfloat16), chunk=16)
    with pytest.raises(ValueError):   # s_final with the wrong batch
        efla.efla_chunk_recurrence(q, k, v, ws, s_final=torch.zeros(1, 3, 16, 32), chunk=16)


def test_workspace_must_share_the_device(host):
    q, k, v, beta = _inputs()
    ws = torch.zeros(1 << 10, dtype=torch.uint8, device="meta")
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd(q, k, v, beta, chunk=16, workspace=ws)
    with pytest.raises(ValueError):
        efla.efla_chunk_recurrence(q, k, v, ws, chunk=16)


def test_varlen_rejects_bad_outputs(host):
    T, H, dk, dv = 40, 2, 16, 16
    q = torch.zeros(T, H, dk, dtype=torch.bfloat16)
    v = torch.zeros(T, H, dv, dtype=torch.bfloat16)
    beta = torch.zeros(T, H, dtype=torch.bfloat16)
    cu = torch.tensor([0, 10, 40], dtype=torch.int32)
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd_varlen(q, q, v, beta, cu, o=torch.zeros(T - 1, H, dv, dtype=torch.bfloat16), chunk=16)
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd_varlen(q, q, v, beta, cu, s_final=torch.zeros(3, H, dk, dv), chunk=16)
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd_varlen(q, q, v, beta, cu.long(), chunk=16)


def test_step_rejects_bad_outputs(host):
    N, H, dk, dv = 4, 2, 16, 32
    q = torch.zeros(N, H, dk, dtype=torch.bfloat16)
    v = torch.zeros(N, H, dv, dtype=torch.bfloat16)
    beta = torch.zeros(N, H, dtype=torch.bfloat16)
    state = torch.zeros(N, H, dk, dv)
    with pytest.raises(ValueError):
        efla.efla_step(q, q, v, beta, state, o=torch.zeros(N, H, dk, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        efla.efla_step(q, q, v, beta, state[:, :, :8])
    with pytest.raises(ValueError):
        efla.prepare_step(q, q, v, beta, state, torch.zeros(N, H + 1, dv, dtype=torch.bfloat16))


def test_prepared_calls_check_shapes(host):
    q, k, v, beta = _inputs()
    ws = torch.zeros(1 << 10, dtype=torch.uint8)
    o = torch.zeros(2, 8, 3, 32, dtype=torch.bfloat16)
    bad_s = torch.zeros(2, 3, 16, 16)
    with pytest.raises(ValueError):
        efla.prepare_chunk_fwd(q, k, v, beta, None, o, bad_s, ws, chunk=16)
    with pytest.raises(ValueError):
        efla.prepare_chunk_stages(q, k, v, beta, None, o[..., :16], None, ws, chunk=16)
    with pytest.raises(ValueError):
        efla.prepare_chunk_bwd(q, k, v, beta, o, None, None, q, k, v[..., :16], beta, None, ws, chunk=16)


def test_training_pair_checks_shapes_and_workspace_device(host):
    q, k, v, beta = _inputs()
    ws = torch.zeros(1 << 10, dtype=torch.uint8)
    o = torch.zeros(2, 8, 3, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd_train(q, k, v, beta, chunk=16, o=o[..., :16], workspace=ws)
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd_train(q, k, v, beta, chunk=16, s_final=torch.zeros(2, 3, 16, 16), workspace=ws)
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd_train(q, k, v, beta, chunk=16, workspace=ws.to("meta"))
    with pytest.raises(ValueError):
        efla.efla_chunk_bwd_train(q, k, v, beta, o[:, :4], ws, chunk=16)          # d_o not shaped like v
    with pytest.raises(ValueError):
        efla.efla_chunk_bwd_train(q, k, v, beta, o, ws, None, torch.zeros(2, 3, 16, 16), chunk=16)
    with pytest.raises(ValueError):
        efla.efla_chunk_bwd_train(q, k, v, beta, o, ws.to("meta"), chunk=16)
    with pytest.raises(ValueError):
        efla.prepare_chunk_train(q, k, v, beta, o, None, o, None, None, q, k, v[..., :16], beta, None, ws, chunk=16)
    with pytest.raises(ValueError):
        efla.prepare_chunk_train(q, k, v, beta, o, None, o[..., :16], None, None, q, k, v, beta, None, ws, chunk=16)
