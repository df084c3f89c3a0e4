"""Python binding of libefla (include/efla.h): argument marshalling only.

Every function takes torch tensors that live on the GPU, checks shapes and
dtypes, and passes raw device pointers plus torch's current HIP stream to the
C ABI of the same name.  All arithmetic happens in the HIP kernels of
``libefla.so``; there is no fallback path.  If the library is missing the first
call raises ``RuntimeError``.

EFLA ("Exact Flow Linear Attention", pages' Method steps 2-3): per (b, h),
alpha_t = (1 - exp(-beta_t ||k_t||^2)) / ||k_t||^2,
S_t = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T, o_t = S_t^T q_t.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libefla.so")

EFLA_F32, EFLA_BF16 = 0, 1
_DTYPES = {torch.float32: EFLA_F32, torch.bfloat16: EFLA_BF16}
_STATUS = {0: "EFLA_OK", 1: "EFLA_ERR_INVALID_ARG", 2: "EFLA_ERR_UNSUPPORTED",
           3: "EFLA_ERR_WORKSPACE", 4: "EFLA_ERR_HIP", 5: "EFLA_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20   # EFLA_NOALLOC_SCRATCH_BYTES of include/efla.h

_lib = None
_vp, _i, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t


class EflaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {efla_status_string(status)}")


def lib() -> ctypes.CDLL:
    """Load libefla.so (built in-tree by build.py); raise if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(or python delta_rule_sequence_efla_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        L.efla_status_string.restype = ctypes.c_char_p
        L.efla_status_string.argtypes = [_i]
        L.efla_chunk_recurrence_kernel.restype = ctypes.c_char_p
        L.efla_chunk_recurrence_kernel.argtypes = [_i, _i, _i, _i]
        L.efla_coeff.restype = _i
        L.efla_coeff.argtypes = [_vp, _vp, _vp, _vp, _i64, _i, _i, _vp]
        L.efla_chunk_fwd_workspace_size.restype = _sz
        L.efla_chunk_fwd_workspace_size.argtypes = [_i, _i, _i64, _i, _i, _i, _i]
        L.efla_chunk_fwd.restype = _i
        L.efla_chunk_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i64, _i, _i, _i,
                                     _i, _vp, _sz, _vp]
        L.efla_chunk_ut_transform.restype = _i
        L.efla_chunk_ut_transform.argtypes = [_vp, _vp, _i, _i, _i64, _i, _i, _i, _vp, _sz, _vp]
        L.efla_chunk_recurrence.restype = _i
        L.efla_chunk_recurrence.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i64, _i, _i,
                                            _i, _i, _vp, _sz, _vp]
        L.efla_step.restype = _i
        L.efla_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
        L.efla_coeff_rule.restype = _i
        L.efla_coeff_rule.argtypes = [_vp, _vp, _vp, _vp, _i64, _i, _i, _i, _vp]
        L.efla_chunk_fwd_rule.restype = _i
        L.efla_chunk_fwd_rule.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i64, _i, _i, _i,
                                          _i, _i, _vp, _sz, _vp]
        L.efla_chunk_ut_transform_rule.restype = _i
        L.efla_chunk_ut_transform_rule.argtypes = [_vp, _vp, _i, _i, _i64, _i, _i, _i, _i, _vp, _sz, _vp]
        L.efla_step_rule.restype = _i
        L.efla_step_rule.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]
        L.efla_chunk_fwd_segmented_workspace_size.restype = _sz
        L.efla_chunk_fwd_segmented_workspace_size.argtypes = [_i, _i, _i64, _i, _i, _i, _i, _i]
        L.efla_chunk_fwd_segmented.restype = _i
        L.efla_chunk_fwd_segmented.argtypes = [_vp] * 7 + [_i, _i, _i64, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]
        L.efla_chunk_bwd_workspace_size.restype = _sz
        L.efla_chunk_bwd_workspace_size.argtypes = [_i, _i, _i64, _i, _i, _i, _i]
        L.efla_chunk_bwd.restype = _i
        L.efla_chunk_bwd.argtypes = [_vp] * 12 + [_i, _i, _i64, _i, _i, _i, _i, _i, _vp, _sz, _vp]
        L.efla_chunk_train_saves_states.restype = _i
        L.efla_chunk_train_saves_states.argtypes = [_i, _i, _i, _i]
        L.efla_chunk_fwd_train.restype = _i
        L.efla_chunk_fwd_train.argtypes = [_vp] * 7 + [_i, _i, _i64, _i, _i, _i, _i, _i, _vp, _sz, _vp]
        L.efla_chunk_bwd_train.restype = _i
        L.efla_chunk_bwd_train.argtypes = [_vp] * 12 + [_i, _i, _i64, _i, _i, _i, _i, _i, _vp, _sz, _vp]
        L.efla_chunk_fwd_varlen_workspace_size.restype = _sz
        L.efla_chunk_fwd_varlen_workspace_size.argtypes = [_i, _i, _i64, _i, _i, _i, _i]
        L.efla_chunk_fwd_noalloc.restype = _i
        L.efla_chunk_fwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i64, _i, _i, _i,
                                             _i, _i, _vp]
        L.efla_chunk_fwd_varlen.restype = _i
        L.efla_chunk_fwd_varlen.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i64, _i, _i,
                                            _i, _i, _i, _vp, _sz, _vp]
        _lib = L
    return _lib


def efla_status_string(status: int) -> str:
    try:
        return lib().efla_status_string(int(status)).decode()
    except RuntimeError:
        return _STATUS.get(int(status), f"status {status}")


def efla_chunk_recurrence_kernel(d_k: int, d_v: int, chunk: int, dtype) -> str:
    """Base name of the recurrence kernel the library launches for these sizes."""
    return lib().efla_chunk_recurrence_kernel(int(d_k), int(d_v), int(chunk), _code(dtype)).decode()


# update rules of include/efla.h: the exact flow, or one explicit Euler step
# (the delta rule), alpha = beta
RULES = {"exact": 0, "euler": 1}


def _rule(rule) -> int:
    if rule not in RULES:
        raise ValueError(f"unknown rule {rule!r}; use 'exact' or 'euler'")
    return RULES[rule]


def _check(status: int, where: str) -> None:
    if status != 0:
        raise EflaError(status, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(*ts, dtype=None):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("EFLA tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("EFLA tensors must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"expected dtype {dtype}, got {t.dtype}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("EFLA tensors must share one device")
    return dev


def _code(dtype) -> int:
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}; use float32 or bfloat16")
    return _DTYPES[dtype]


def _want(t, shape, name: str, dtype=None) -> None:
    """A caller-supplied output or state must have exactly the shape (and
    dtype) the kernels index it with: the library only sees a pointer."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _ws(workspace, dev, name: str = "workspace") -> int:
    """Byte size of a workspace tensor, which must be on the call's device."""
    if workspace is None:
        return 0
    if _dev(workspace) != dev:
        raise ValueError(f"{name} must live on {dev}")
    return workspace.numel() * workspace.element_size()


def efla_coeff(k: torch.Tensor, beta: torch.Tensor, want_lambda: bool = True, rule: str = "exact"):
    """lambda = ||k||^2 and alpha per key row; k [..., d_k], beta [...] -> fp32."""
    dev = _dev(k, beta, dtype=k.dtype)
    n = k.numel() // k.shape[-1]
    if beta.numel() != n:
        raise ValueError("beta needs one value per key row")
    alpha = torch.empty(k.shape[:-1], dtype=torch.float32, device=dev)
    lam = torch.empty_like(alpha) if want_lambda else None
    with torch.cuda.device(dev):
        _check(lib().efla_coeff_rule(_p(k), _p(beta), _p(lam), _p(alpha), n, k.shape[-1],
                                     _code(k.dtype), _rule(rule), _stream(dev)), "efla_coeff")
    return lam, alpha


def efla_chunk_fwd_workspace_size(B, H, L, d_k, d_v, chunk, dtype) -> int:
    return int(lib().efla_chunk_fwd_workspace_size(B, H, L, d_k, d_v, chunk, _code(dtype)))


def _chunk_shapes(q, k, v, beta, s0):
    _dev(q, k, v, beta, s0)  # one device for inputs and the initial state
    if k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected q, k [B,L,H,dk], v [B,L,H,dv], beta [B,L,H]")
    B, L, H, dk = k.shape
    dv = v.shape[-1]
    if q.shape != k.shape or v.shape[:3] != (B, L, H) or beta.shape != (B, L, H):
        raise ValueError("expected q, k [B,L,H,dk], v [B,L,H,dv], beta [B,L,H]")
    if s0 is not None and (s0.shape != (B, H, dk, dv) or s0.dtype != torch.float32):
        raise ValueError("s0 must be float32 [B,H,dk,dv]")
    return B, L, H, dk, dv


def _fwd_outs(o, s_final, B, L, H, dk, dv, dtype, ref=None) -> None:
    _dev(ref, o, s_final)
    _want(o, (B, L, H, dv), "o", dtype)
    _want(s_final, (B, H, dk, dv), "s_final", torch.float32)


def alloc_workspace(B, H, L, d_k, d_v, chunk, dtype, device) -> torch.Tensor:
    n = efla_chunk_fwd_workspace_size(B, H, L, d_k, d_v, chunk, dtype)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def efla_chunk_fwd(q, k, v, beta, s0=None, chunk: int = 64, o=None, s_final=None,
                   workspace=None, want_final: bool = True, rule: str = "exact"):
    """Chunked EFLA forward.  Returns (o [B,L,H,dv] in q's dtype, S_L fp32 or None)."""
    dev = _dev(q, k, v, beta, o, workspace, dtype=None)
    _dev(q, k, v, beta, o, dtype=q.dtype)
    _dev(s0, s_final, dtype=torch.float32)
    B, L, H, dk, dv = _chunk_shapes(q, k, v, beta, s0)
    _fwd_outs(o, s_final, B, L, H, dk, dv, q.dtype, q)
    if o is None:
        o = torch.empty((B, L, H, dv), dtype=q.dtype, device=dev)
    if s_final is None and want_final:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(B, H, L, dk, dv, chunk, q.dtype, dev)
    nws = _ws(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib().efla_chunk_fwd_rule(_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(o), _p(s_final),
                                         B, H, L, dk, dv, chunk, _code(q.dtype), _rule(rule), _p(workspace),
                                         nws, _stream(dev)), "efla_chunk_fwd")
    return o, s_final


def efla_chunk_fwd_noalloc(q, k, v, beta, s0=None, chunk: int = 64, o=None, s_final=None,
                           want_final: bool = True, rule: str = "exact"):
    """efla_chunk_fwd with the library's fixed per-GPU scratch instead of a
    workspace (no device allocation inside the call; o and s_final are
    allocated here unless given).  Calls that overlap on one GPU race."""
    dev = _dev(q, k, v, beta, o, dtype=q.dtype)
    _dev(s0, s_final, dtype=torch.float32)
    B, L, H, dk, dv = _chunk_shapes(q, k, v, beta, s0)
    _fwd_outs(o, s_final, B, L, H, dk, dv, q.dtype, q)
    if o is None:
        o = torch.empty((B, L, H, dv), dtype=q.dtype, device=dev)
    if s_final is None and want_final:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check(lib().efla_chunk_fwd_noalloc(_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(o), _p(s_final),
                                            B, H, L, dk, dv, chunk, _code(q.dtype), _rule(rule), _stream(dev)),
               "efla_chunk_fwd_noalloc")
    return o, s_final


def efla_chunk_ut_transform(k, beta, chunk: int = 64, workspace=None, rule: str = "exact"):
    """Stage 1 only: per-chunk T into the workspace (returned as [B,H,NC,C,C] view)."""
    dev = _dev(k, beta, dtype=k.dtype)
    if k.dim() != 4:
        raise ValueError("k must be [B,L,H,dk]")
    B, L, H, dk = k.shape
    _want(beta, (B, L, H), "beta")
    if workspace is None:
        workspace = alloc_workspace(B, H, L, dk, 16, chunk, k.dtype, dev)
    nws = _ws(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib().efla_chunk_ut_transform_rule(_p(k), _p(beta), B, H, L, dk, chunk, _code(k.dtype),
                                                  _rule(rule), _p(workspace), nws, _stream(dev)),
               "efla_chunk_ut_transform")
    nc = (L + chunk - 1) // chunk
    n = B * H * nc * chunk * chunk
    return workspace, workspace[: n * k.element_size()].view(k.dtype).view(B, H, nc, chunk, chunk)


def efla_chunk_recurrence(q, k, v, workspace, s0=None, chunk: int = 64, o=None, s_final=None,
                          want_final: bool = True):
    """Stage 2 only, reading T from a workspace filled by efla_chunk_ut_transform."""
    dev = _dev(q, k, v, o, dtype=q.dtype)
    _dev(q, s0, s_final)
    _dev(s0, s_final, dtype=torch.float32)
    if k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected q, k [B,L,H,dk], v [B,L,H,dv]")
    B, L, H, dk = k.shape
    dv = v.shape[-1]
    _want(q, (B, L, H, dk), "q")
    _want(v, (B, L, H, dv), "v")
    _want(s0, (B, H, dk, dv), "s0")
    _fwd_outs(o, s_final, B, L, H, dk, dv, q.dtype, q)
    if o is None:
        o = torch.empty((B, L, H, dv), dtype=q.dtype, device=dev)
    if s_final is None and want_final:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    nws = _ws(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib().efla_chunk_recurrence(_p(q), _p(k), _p(v), _p(s0), _p(o), _p(s_final), B, H, L,
                                           dk, dv, chunk, _code(q.dtype), _p(workspace),
                                           nws, _stream(dev)), "efla_chunk_recurrence")
    return o, s_final


COMPUTE_UNITS = 256  # MI355X


def default_segments(B, H, L, d_v, chunk) -> int:
    """Segments per sequence for efla_chunk_fwd_segmented: enough recurrence
    workgroups (B * H * d_v / 32 per segment) to reach the compute units."""
    per_seg = max(1, B * H * max(1, d_v // 32))
    nc = max(1, (L + chunk - 1) // chunk)
    return max(1, min(nc, COMPUTE_UNITS // per_seg))


def efla_chunk_fwd_segmented_workspace_size(B, H, L, d_k, d_v, chunk, segments, dtype) -> int:
    return int(lib().efla_chunk_fwd_segmented_workspace_size(B, H, L, d_k, d_v, chunk, segments, _code(dtype)))


def efla_chunk_fwd_segmented(q, k, v, beta, s0=None, chunk: int = 64, segments=None, o=None, s_final=None,
                             workspace=None, want_final: bool = True, rule: str = "exact"):
    """efla_chunk_fwd with each sequence cut into `segments` runs that proceed
    in parallel (None: default_segments).  Same results up to rounding."""
    dev = _dev(q, k, v, beta, o, workspace, dtype=None)
    _dev(q, k, v, beta, o, dtype=q.dtype)
    _dev(s0, s_final, dtype=torch.float32)
    B, L, H, dk, dv = _chunk_shapes(q, k, v, beta, s0)
    _fwd_outs(o, s_final, B, L, H, dk, dv, q.dtype, q)
    if segments is None:
        segments = default_segments(B, H, L, dv, chunk)
    if o is None:
        o = torch.empty((B, L, H, dv), dtype=q.dtype, device=dev)
    if s_final is None and want_final:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if workspace is None:
        n = efla_chunk_fwd_segmented_workspace_size(B, H, L, dk, dv, chunk, segments, q.dtype)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    nws = _ws(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib().efla_chunk_fwd_segmented(_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(o), _p(s_final), B, H, L,
                                              dk, dv, chunk, segments, _code(q.dtype), _rule(rule), _p(workspace),
                                              nws, _stream(dev)), "efla_chunk_fwd_segmented")
    return o, s_final


def prepare_chunk_fwd_segmented(q, k, v, beta, s0, o, s_final, workspace, chunk: int = 64, segments: int = 1,
                                rule: str = "exact"):
    dev = _dev(q, k, v, beta, o, dtype=q.dtype)
    _dev(s0, s_final, dtype=torch.float32)
    B, L, H, dk, dv = _chunk_shapes(q, k, v, beta, s0)
    _fwd_outs(o, s_final, B, L, H, dk, dv, q.dtype, q)
    nws = _ws(workspace, dev)
    return PreparedCall(lib().efla_chunk_fwd_segmented,
                        (_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(o), _p(s_final), B, H, L, dk, dv, chunk,
                         segments, _code(q.dtype), _rule(rule), _p(workspace), nws, _stream(dev)),
                        "efla_chunk_fwd_segmented", (q, k, v, beta, s0, o, s_final, workspace))


def efla_chunk_bwd_workspace_size(B, H, L, d_k, d_v, chunk, dtype) -> int:
    return int(lib().efla_chunk_bwd_workspace_size(B, H, L, d_k, d_v, chunk, _code(dtype)))


def efla_chunk_bwd(q, k, v, beta, d_o, s0=None, ds_final=None, chunk: int = 64, rule: str = "exact",
                   want_ds0: bool = True, workspace=None):
    """Gradients through efla_chunk_fwd for dLoss/do = d_o and dLoss/dS_L =
    ds_final (None: zero).  Returns (dq, dk, dv, dbeta, ds0) in the input
    dtype (ds0 fp32 [B,H,dk,dv], or None when want_ds0 is False)."""
    dev = _dev(q, k, v, beta, d_o, workspace, dtype=None)
    _dev(q, k, v, beta, d_o, dtype=q.dtype)
    _dev(s0, ds_final, dtype=torch.float32)
    B, L, H, dk, dv = _chunk_shapes(q, k, v, beta, s0)
    if d_o.shape != v.shape:
        raise ValueError("d_o must have the shape of v")
    if ds_final is not None and ds_final.shape != (B, H, dk, dv):
        raise ValueError("ds_final must be float32 [B,H,dk,dv]")
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    gb = torch.empty_like(beta)
    gs0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_ds0 else None
    if workspace is None:
        n = efla_chunk_bwd_workspace_size(B, H, L, dk, dv, chunk, q.dtype)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    nws = _ws(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib().efla_chunk_bwd(_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(d_o), _p(ds_final), _p(gq), _p(gk),
                                    _p(gv), _p(gb), _p(gs0), B, H, L, dk, dv, chunk, _code(q.dtype), _rule(rule),
                                    _p(workspace), nws, _stream(dev)), "efla_chunk_bwd")
    return gq, gk, gv, gb, gs0


def efla_chunk_train_saves_states(d_k: int, d_v: int, chunk: int, dtype) -> bool:
    return bool(lib().efla_chunk_train_saves_states(d_k, d_v, chunk, _code(dtype)))


def efla_chunk_fwd_train(q, k, v, beta, s0=None, chunk: int = 64, o=None, s_final=None, workspace=None,
                         want_final: bool = True, rule: str = "exact"):
    """efla_chunk_fwd that also leaves in ``workspace`` (bytes of
    efla_chunk_bwd_workspace_size; allocated here when None) what
    efla_chunk_bwd_train reads.  Returns (o, S_L or None, workspace)."""
    dev = _dev(q, k, v, beta, o, workspace, dtype=None)
    _dev(q, k, v, beta, o, dtype=q.dtype)
    _dev(s0, s_final, dtype=torch.float32)
    B, L, H, dk, dv = _chunk_shapes(q, k, v, beta, s0)
    _fwd_outs(o, s_final, B, L, H, dk, dv, q.dtype, q)
    if o is None:
        o = torch.empty((B, L, H, dv), dtype=q.dtype, device=dev)
    if s_final is None and want_final:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if workspace is None:
        n = efla_chunk_bwd_workspace_size(B, H, L, dk, dv, chunk, q.dtype)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    nws = _ws(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib().efla_chunk_fwd_train(_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(o), _p(s_final),
                                          B, H, L, dk, dv, chunk, _code(q.dtype), _rule(rule), _p(workspace),
                                          nws, _stream(dev)), "efla_chunk_fwd_train")
    return o, s_final, workspace


def efla_chunk_bwd_train(q, k, v, beta, d_o, workspace, s0=None, ds_final=None, chunk: int = 64,
                         rule: str = "exact", want_ds0: bool = True):
    """efla_chunk_bwd after efla_chunk_fwd_train (same inputs, sizes, rule
    and the workspace it filled).  Returns (dq, dk, dv, dbeta, ds0)."""
    dev = _dev(q, k, v, beta, d_o, workspace, dtype=None)
    _dev(q, k, v, beta, d_o, dtype=q.dtype)
    _dev(s0, ds_final, dtype=torch.float32)
    B, L, H, dk, dv = _chunk_shapes(q, k, v, beta, s0)
    if d_o.shape != v.shape:
        raise ValueError("d_o must have the shape of v")
    if ds_final is not None and ds_final.shape != (B, H, dk, dv):
        raise ValueError("ds_final must be float32 [B,H,dk,dv]")
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    gb = torch.empty_like(beta)
    gs0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_ds0 else None
    nws = _ws(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib().efla_chunk_bwd_train(_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(d_o), _p(ds_final), _p(gq),
                                          _p(gk), _p(gv), _p(gb), _p(gs0), B, H, L, dk, dv, chunk, _code(q.dtype),
                                          _rule(rule), _p(workspace), nws, _stream(dev)), "efla_chunk_bwd_train")
    return gq, gk, gv, gb, gs0


def efla_chunk_fwd_varlen_workspace_size(N, H, T, d_k, d_v, chunk, dtype) -> int:
    return int(lib().efla_chunk_fwd_varlen_workspace_size(N, H, T, d_k, d_v, chunk, _code(dtype)))


def _varlen_shapes(q, k, v, beta, cu_seqlens, s0):
    _dev(q, k, v, beta, cu_seqlens, s0)
    if k.dim() == 4 and k.shape[0] == 1:   # [1, T, H, d] packed layout
        q, k, v, beta = q[0], k[0], v[0], beta[0]
    T, H, dk = k.shape
    dv = v.shape[-1]
    if q.shape != k.shape or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("expected q, k [T,H,dk], v [T,H,dv], beta [T,H] (or with a leading 1)")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of N+1 offsets")
    N = cu_seqlens.numel() - 1
    if s0 is not None and (s0.shape != (N, H, dk, dv) or s0.dtype != torch.float32):
        raise ValueError("s0 must be float32 [N,H,dk,dv]")
    return N, T, H, dk, dv


def _varlen_outs(o, s_final, v, N, H, dk, dv, dtype) -> None:
    _dev(v, o, s_final)
    _want(o, v.shape, "o", dtype)
    _want(s_final, (N, H, dk, dv), "s_final", torch.float32)


def efla_chunk_fwd_varlen(q, k, v, beta, cu_seqlens, s0=None, chunk: int = 64, o=None, s_final=None,
                          workspace=None, want_final: bool = True, rule: str = "exact"):
    """Chunked forward over a packed variable-length batch: q, k [T,H,dk],
    v [T,H,dv], beta [T,H] (a leading batch dim of 1 is accepted), int32
    device offsets cu_seqlens [N+1].  Returns (o shaped like v, S fp32 [N,H,dk,dv])."""
    dev = _dev(q, k, v, beta, o, workspace, cu_seqlens, dtype=None)
    _dev(q, k, v, beta, o, dtype=q.dtype)
    _dev(s0, s_final, dtype=torch.float32)
    N, T, H, dk, dv = _varlen_shapes(q, k, v, beta, cu_seqlens, s0)
    _varlen_outs(o, s_final, v, N, H, dk, dv, q.dtype)
    if o is None:
        o = torch.empty(v.shape, dtype=q.dtype, device=dev)
    if s_final is None and want_final:
        s_final = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if workspace is None:
        n = efla_chunk_fwd_varlen_workspace_size(N, H, T, dk, dv, chunk, q.dtype)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    nws = _ws(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib().efla_chunk_fwd_varlen(_p(q), _p(k), _p(v), _p(beta), _p(cu_seqlens), N, _p(s0), _p(o),
                                           _p(s_final), H, T, dk, dv, chunk, _code(q.dtype), _rule(rule),
                                           _p(workspace), nws, _stream(dev)),
               "efla_chunk_fwd_varlen")
    return o, s_final


def prepare_chunk_fwd_varlen(q, k, v, beta, cu_seqlens, s0, o, s_final, workspace, chunk: int = 64,
                             rule: str = "exact"):
    dev = _dev(q, k, v, beta, o, dtype=q.dtype)
    _dev(s0, s_final, dtype=torch.float32)
    N, T, H, dk, dv = _varlen_shapes(q, k, v, beta, cu_seqlens, s0)
    _dev(q, cu_seqlens)
    _varlen_outs(o, s_final, v, N, H, dk, dv, q.dtype)
    nws = _ws(workspace, dev)
    return PreparedCall(lib().efla_chunk_fwd_varlen,
                        (_p(q), _p(k), _p(v), _p(beta), _p(cu_seqlens), N, _p(s0), _p(o), _p(s_final), H, T,
                         dk, dv, chunk, _code(q.dtype), _rule(rule), _p(workspace), nws,
                         _stream(dev)),
                        "efla_chunk_fwd_varlen", (q, k, v, beta, cu_seqlens, s0, o, s_final, workspace))


def efla_step(q, k, v, beta, state, o=None, rule: str = "exact"):
    """One decode step in place on state [N,H,dk,dv] (fp32).  Returns o [N,H,dv]."""
    dev = _dev(q, k, v, beta, o, dtype=q.dtype)
    _dev(state, dtype=torch.float32)
    N, H, dk = k.shape
    dv = v.shape[-1]
    if q.shape != k.shape or v.shape[:2] != (N, H) or beta.shape != (N, H) \
            or state.shape != (N, H, dk, dv):
        raise ValueError("expected q, k [N,H,dk], v [N,H,dv], beta [N,H], state [N,H,dk,dv]")
    _want(o, (N, H, dv), "o", q.dtype)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    with torch.cuda.device(dev):
        _check(lib().efla_step_rule(_p(q), _p(k), _p(v), _p(beta), _p(state), _p(o), N, H, dk, dv,
                                    _code(q.dtype), _rule(rule), _stream(dev)), "efla_step")
    return o


class PreparedCall:
    """A C-ABI call with its arguments marshalled once (for tight timing loops).

    Calling it re-issues the same launch on the stream captured at preparation;
    the tensors passed to ``prepare_*`` must stay alive and unchanged in shape.
    """

    def __init__(self, fn, args, where: str, keep):
        self._fn, self._args, self._where, self._keep = fn, args, where, keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != 0:
            raise EflaError(st, self._where)


def prepare_chunk_stages(q, k, v, beta, s0, o, s_final, workspace, chunk: int = 64, rule: str = "exact"):
    """(ut_transform, recurrence) prepared calls: together exactly efla_chunk_fwd."""
    dev = _dev(q, k, v, beta, o, dtype=q.dtype)
    _dev(s0, s_final, dtype=torch.float32)
    B, L, H, dk, dv = _chunk_shapes(q, k, v, beta, s0)
    _fwd_outs(o, s_final, B, L, H, dk, dv, q.dtype, q)
    code = _code(q.dtype)
    stream = _stream(dev)
    ws, nbytes = _p(workspace), _ws(workspace, dev)
    ut = PreparedCall(lib().efla_chunk_ut_transform_rule,
                      (_p(k), _p(beta), B, H, L, dk, chunk, code, _rule(rule), ws, nbytes, stream),
                      "efla_chunk_ut_transform", (k, beta, workspace))
    rec = PreparedCall(lib().efla_chunk_recurrence,
                       (_p(q), _p(k), _p(v), _p(s0), _p(o), _p(s_final), B, H, L, dk, dv, chunk,
                        code, ws, nbytes, stream),
                       "efla_chunk_recurrence", (q, k, v, s0, o, s_final, workspace))
    return ut, rec


def prepare_chunk_fwd(q, k, v, beta, s0, o, s_final, workspace, chunk: int = 64, rule: str = "exact"):
    dev = _dev(q, k, v, beta, o, dtype=q.dtype)
    _dev(s0, s_final, dtype=torch.float32)
    B, L, H, dk, dv = _chunk_shapes(q, k, v, beta, s0)
    _fwd_outs(o, s_final, B, L, H, dk, dv, q.dtype, q)
    nws = _ws(workspace, dev)
    return PreparedCall(lib().efla_chunk_fwd_rule,
                        (_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(o), _p(s_final), B, H, L, dk, dv,
                         chunk, _code(q.dtype), _rule(rule), _p(workspace), nws, _stream(dev)),
                        "efla_chunk_fwd", (q, k, v, beta, s0, o, s_final, workspace))


def prepare_chunk_bwd(q, k, v, beta, d_o, s0, ds_final, dq, dk, dv, dbeta, ds0, workspace, chunk: int = 64,
                      rule: str = "exact"):
    dev = _dev(q, k, v, beta, d_o, dq, dk, dv, dbeta, dtype=q.dtype)
    _dev(s0, ds_final, ds0, dtype=torch.float32)
    B, L, H, d_k, d_v = _chunk_shapes(q, k, v, beta, s0)
    for t, like, name in ((d_o, v, "d_o"), (dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv"), (dbeta, beta, "dbeta")):
        _want(t, like.shape, name)
    _want(ds_final, (B, H, d_k, d_v), "ds_final")
    _want(ds0, (B, H, d_k, d_v), "ds0")
    nws = _ws(workspace, dev)
    return PreparedCall(lib().efla_chunk_bwd,
                        (_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(d_o), _p(ds_final), _p(dq), _p(dk), _p(dv),
                         _p(dbeta), _p(ds0), B, H, L, d_k, d_v, chunk, _code(q.dtype), _rule(rule), _p(workspace),
                         nws, _stream(dev)),
                        "efla_chunk_bwd", (q, k, v, beta, d_o, s0, ds_final, dq, dk, dv, dbeta, ds0, workspace))


def prepare_chunk_train(q, k, v, beta, d_o, s0, o, s_final, ds_final, dq, dk, dv, dbeta, ds0, workspace,
                        chunk: int = 64, rule: str = "exact"):
    """(forward, backward) prepared calls of the training pair sharing ``workspace``."""
    dev = _dev(q, k, v, beta, d_o, o, dq, dk, dv, dbeta, dtype=q.dtype)
    _dev(s0, s_final, ds_final, ds0, dtype=torch.float32)
    B, L, H, d_k, d_v = _chunk_shapes(q, k, v, beta, s0)
    _fwd_outs(o, s_final, B, L, H, d_k, d_v, q.dtype, q)
    for t, like, name in ((d_o, v, "d_o"), (dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv"), (dbeta, beta, "dbeta")):
        _want(t, like.shape, name)
    _want(ds_final, (B, H, d_k, d_v), "ds_final")
    _want(ds0, (B, H, d_k, d_v), "ds0")
    code, ws, nws, stream = _code(q.dtype), _p(workspace), _ws(workspace, dev), _stream(dev)
    fwd = PreparedCall(lib().efla_chunk_fwd_train,
                       (_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(o), _p(s_final), B, H, L, d_k, d_v, chunk, code,
                        _rule(rule), ws, nws, stream),
                       "efla_chunk_fwd_train", (q, k, v, beta, s0, o, s_final, workspace))
    bwd = PreparedCall(lib().efla_chunk_bwd_train,
                       (_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(d_o), _p(ds_final), _p(dq), _p(dk), _p(dv),
                        _p(dbeta), _p(ds0), B, H, L, d_k, d_v, chunk, code, _rule(rule), ws, nws, stream),
                       "efla_chunk_bwd_train", (q, k, v, beta, d_o, s0, ds_final, dq, dk, dv, dbeta, ds0, workspace))
    return fwd, bwd


def prepare_step(q, k, v, beta, state, o, rule: str = "exact"):
    dev = _dev(q, k, v, beta, o, dtype=q.dtype)
    _dev(state, dtype=torch.float32)
    N, H, dk = k.shape
    dv = v.shape[-1]
    if q.shape != k.shape or v.shape[:2] != (N, H) or beta.shape != (N, H):
        raise ValueError("expected q, k [N,H,dk], v [N,H,dv], beta [N,H]")
    _want(state, (N, H, dk, dv), "state")
    _want(o, (N, H, dv), "o")
    return PreparedCall(lib().efla_step_rule,
                        (_p(q), _p(k), _p(v), _p(beta), _p(state), _p(o), N, H, dk, dv,
                         _code(q.dtype), _rule(rule), _stream(dev)),
                        "efla_step", (q, k, v, beta, state, o))
