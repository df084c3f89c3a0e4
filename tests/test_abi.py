"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/efla.h declares, and rejects bad arguments before
launching anything."""
import ctypes
import os
import re

import pytest
import torch

from delta_rule_sequence_efla_amd import efla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "efla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(efla_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["efla_coeff", "efla_chunk_fwd_workspace_size", "efla_chunk_fwd", "efla_step",
                     "efla_status_string", "efla_chunk_ut_transform", "efla_chunk_recurrence"]:
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = efla.lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"libefla.so does not export {name}"


def test_status_strings():
    for code, prefix in [(0, "EFLA_OK"), (1, "EFLA_ERR_INVALID_ARG"), (2, "EFLA_ERR_UNSUPPORTED"),
                         (3, "EFLA_ERR_WORKSPACE"), (4, "EFLA_ERR_HIP"), (5, "EFLA_ERR_SCRATCH")]:
        assert efla.efla_status_string(code).startswith(prefix)
    assert efla.efla_status_string(99) == "EFLA_ERR_UNKNOWN"


def test_recurrence_kernel_names():
    """The kernel-name query follows the dispatch rule and launches nothing."""
    import torch
    name = efla.efla_chunk_recurrence_kernel
    assert name(128, 128, 64, torch.bfloat16) == "recurrence_split_kernel"
    assert name(64, 64, 64, torch.bfloat16) == "recurrence_split_kernel"
    assert name(128, 128, 32, torch.bfloat16) == "recurrence_roles_kernel"  # chunk 32
    assert name(128, 16, 64, torch.bfloat16) == "recurrence_roles_kernel"   # one 16-column tile
    assert name(16, 64, 16, torch.bfloat16) == "recurrence_kernel"       # d_k 16, chunk 16
    assert name(128, 128, 64, torch.float32) == "recurrence_kernel"
    assert name(48, 128, 64, torch.bfloat16) == "unsupported"
    assert name(128, 128, 128, torch.bfloat16) == "unsupported"


def test_workspace_size():
    f = efla.efla_chunk_fwd_workspace_size
    # 1.3B-shaped layer: 4*16 sequences x 64 chunks x 64x64 bf16
    assert f(4, 16, 4096, 128, 128, 64, torch.bfloat16) == 4 * 16 * 64 * 64 * 64 * 2
    assert f(1, 1, 65, 16, 16, 16, torch.float32) == 5 * 16 * 16 * 4  # ragged: 5 chunks
    assert f(1, 1, 0, 16, 16, 16, torch.float32) == 0
    assert f(1, 1, 64, 24, 16, 16, torch.float32) == 0    # unsupported d_k
    assert f(1, 1, 64, 16, 16, 48, torch.float32) == 0    # unsupported chunk
    assert f(0, 1, 64, 16, 16, 16, torch.float32) == 0


def test_validation_happens_before_any_launch():
    L = efla.lib()
    nul = None
    # unsupported sizes
    assert L.efla_chunk_fwd(nul, nul, nul, nul, nul, nul, nul, 1, 1, 64, 24, 16, 16, 0, nul, 0, nul) == 2
    assert L.efla_chunk_fwd(nul, nul, nul, nul, nul, nul, nul, 1, 1, 64, 16, 16, 8, 0, nul, 0, nul) == 2
    assert L.efla_step(nul, nul, nul, nul, nul, nul, 1, 1, 16, 200, 1, nul) == 2
    assert L.efla_coeff(nul, nul, nul, nul, 5, 12, 0, nul) == 2
    # invalid arguments
    assert L.efla_chunk_fwd(nul, nul, nul, nul, nul, nul, nul, 0, 1, 64, 16, 16, 16, 0, nul, 0, nul) == 1
    assert L.efla_chunk_fwd(nul, nul, nul, nul, nul, nul, nul, 1, 1, -1, 16, 16, 16, 0, nul, 0, nul) == 1
    assert L.efla_chunk_fwd(nul, nul, nul, nul, nul, nul, nul, 1, 1, 64, 16, 16, 16, 7, nul, 0, nul) == 1
    assert L.efla_chunk_fwd(nul, nul, nul, nul, nul, nul, nul, 1, 1, 64, 16, 16, 16, 0, nul, 0, nul) == 1
    assert L.efla_step(nul, nul, nul, nul, nul, nul, 2, 2, 16, 16, 0, nul) == 1
    assert L.efla_coeff(nul, nul, nul, nul, 5, 16, 0, nul) == 1
    assert L.efla_coeff(nul, nul, nul, nul, -1, 16, 0, nul) == 1
    # workspace too small (pointers are never dereferenced: validation fails first)
    fake = ctypes.c_void_p(4096)
    assert L.efla_chunk_fwd(fake, fake, fake, fake, nul, fake, nul, 1, 1, 64, 16, 16, 16, 0,
                            nul, 0, nul) == 3
    assert L.efla_chunk_fwd(fake, fake, fake, fake, nul, fake, nul, 1, 1, 64, 16, 16, 16, 0,
                            fake, 1023, nul) == 3
    # misaligned q
    odd = ctypes.c_void_p(4098)
    assert L.efla_chunk_fwd(odd, fake, fake, fake, nul, fake, nul, 1, 1, 64, 16, 16, 16, 0,
                            fake, 4096, nul) == 1
    # nothing to do is success without a launch
    assert L.efla_step(nul, nul, nul, nul, nul, nul, 0, 4, 16, 16, 0, nul) == 0
    assert L.efla_coeff(nul, nul, nul, nul, 0, 16, 0, nul) == 0
    assert L.efla_chunk_fwd(nul, nul, nul, nul, nul, nul, nul, 1, 1, 0, 16, 16, 16, 0, nul, 0, nul) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(efla, "_lib", None)
    monkeypatch.setattr(efla, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        efla.lib()


def test_binding_rejects_host_tensors():
    x = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        efla.efla_chunk_fwd(x, x, x, torch.zeros(1, 4, 1), chunk=16)


def test_product_package_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "delta_rule_sequence_efla_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "efla_oracle" not in text, f


def test_rule_is_validated_first():
    """An update rule other than EFLA_RULE_EXACT / EFLA_RULE_EULER is
    EFLA_ERR_INVALID_ARG on every _rule entry point, before size checks and
    before the empty-input early return."""
    L = efla.lib()
    nul = None
    for rule, want in [(0, 2), (1, 2), (2, 1), (-1, 1)]:
        # sizes that are unsupported under a valid rule (d_k 24 / d_v 200)
        assert L.efla_chunk_fwd_rule(nul, nul, nul, nul, nul, nul, nul, 1, 1, 64, 24, 16, 16, 0, rule,
                                     nul, 0, nul) == want
        assert L.efla_chunk_ut_transform_rule(nul, nul, 1, 1, 64, 24, 16, 0, rule, nul, 0, nul) == want
        assert L.efla_step_rule(nul, nul, nul, nul, nul, nul, 1, 1, 16, 200, 1, rule, nul) == want
        assert L.efla_coeff_rule(nul, nul, nul, nul, 5, 12, 0, rule, nul) == want
    # empty inputs: OK under a valid rule, still rejected under a bad one
    assert L.efla_coeff_rule(nul, nul, nul, nul, 0, 16, 0, 1, nul) == 0
    assert L.efla_coeff_rule(nul, nul, nul, nul, 0, 16, 0, 3, nul) == 1
    assert L.efla_step_rule(nul, nul, nul, nul, nul, nul, 0, 4, 16, 16, 0, 1, nul) == 0
    assert L.efla_step_rule(nul, nul, nul, nul, nul, nul, 0, 4, 16, 16, 0, 3, nul) == 1
    assert efla.RULES == {"exact": 0, "euler": 1}
    with pytest.raises(ValueError):
        efla._rule("rk4")


def test_varlen_workspace_size_and_validation():
    f = efla.efla_chunk_fwd_varlen_workspace_size
    # H x (floor(T / C) + N) slots of C x C (256-byte aligned), then the
    # schedule: one int32 per sequence, aligned up to 256 bytes
    assert f(3, 2, 100, 16, 16, 16, torch.float32) == 2 * (6 + 3) * 16 * 16 * 4 + 256
    assert f(16, 16, 16384, 128, 128, 64, torch.bfloat16) == 16 * (256 + 16) * 64 * 64 * 2 + 256
    assert f(65, 1, 64, 16, 16, 16, torch.float32) == (4 + 65) * 16 * 16 * 4 + 512
    assert f(0, 2, 100, 16, 16, 16, torch.float32) == 0
    assert f(3, 2, 100, 24, 16, 16, torch.float32) == 0
    assert f(3, 2, 2 ** 31, 16, 16, 16, torch.float32) == 0
    L = efla.lib()
    nul = None
    fake = 4096  # never dereferenced: every case below returns before a launch

    def call(N=2, H=1, T=64, dk=16, dv=16, C=16, dt=0, rule=0, cu=fake, q=fake, ws=nul, wsb=0):
        return L.efla_chunk_fwd_varlen(q, q, q, q, cu, N, nul, q, nul, H, T, dk, dv, C, dt, rule, ws, wsb, nul)

    assert call(N=-1) == 1 and call(H=0) == 1 and call(T=-1) == 1 and call(dt=5) == 1 and call(rule=2) == 1
    assert call(dk=24) == 2 and call(C=48) == 2 and call(T=2 ** 31) == 2
    assert call(N=0, cu=nul, q=nul) == 0          # no sequences: nothing to do
    assert call(cu=nul) == 1                      # offsets missing
    assert call(q=nul) == 1                       # tokens but no inputs
    assert call(q=fake + 8) == 1                  # misaligned
    assert call() == 3                            # no workspace
    assert call(ws=fake, wsb=10) == 3             # too small


def test_backward_workspace_size_and_validation():
    f = efla.efla_chunk_bwd_workspace_size
    assert f(1, 1, 0, 16, 16, 16, torch.float32) == 0
    assert f(1, 1, 64, 24, 16, 16, torch.float32) == 0
    # 1.3B shape: T (bf16), X, P (fp32), a, chunk states (bf16), their gradients (fp32)
    # and the effective queries Q - P T K (bf16)
    slots = 4 * 16 * 64
    want = slots * (64 * 64 * 2 + 2 * 64 * 64 * 4 + 64 * 4 + 128 * 128 * 2 + 128 * 128 * 4 + 64 * 128 * 2)
    assert f(4, 16, 4096, 128, 128, 64, torch.bfloat16) == want
    # float32: T and the states in float32
    want32 = slots * (64 * 64 * 4 + 2 * 64 * 64 * 4 + 64 * 4 + 128 * 128 * 4 + 128 * 128 * 4)
    assert f(4, 16, 4096, 128, 128, 64, torch.float32) == want32
    L = efla.lib()
    nul, fake = None, 4096

    def call(B=1, L_=64, dk=16, C=16, rule=0, p=fake, ws=nul, wsb=0, ds0=nul):
        return L.efla_chunk_bwd(p, p, p, p, nul, p, nul, p, p, p, p, ds0, B, 1, L_, dk, 16, C, 0, rule, ws, wsb, nul)

    assert call(rule=3) == 1 and call(B=0) == 1 and call(dk=24) == 2 and call(C=48) == 2
    assert call(p=nul) == 1 and call(p=fake + 4) == 1
    assert call() == 3 and call(ws=fake, wsb=16) == 3
    assert call(L_=0, p=nul) == 0               # nothing to do, no ds0 wanted


def test_training_pair_query_and_validation():
    """The training pair stores chunk states only for the shapes whose split
    recurrence and bf16 backward kernels both apply; both calls validate like
    efla_chunk_fwd / efla_chunk_bwd, against the backward workspace size."""
    saves = efla.efla_chunk_train_saves_states
    assert saves(128, 128, 64, torch.bfloat16) and saves(64, 64, 64, torch.bfloat16)
    assert saves(128, 64, 64, torch.bfloat16) and saves(64, 128, 64, torch.bfloat16)
    assert not saves(128, 128, 64, torch.float32)       # fp32: no split recurrence
    assert not saves(128, 128, 32, torch.bfloat16)      # chunk 32
    assert not saves(32, 128, 64, torch.bfloat16)       # d_k 32
    assert not saves(128, 16, 64, torch.bfloat16)       # d_v below one value block
    assert not saves(48, 128, 64, torch.bfloat16)       # unsupported size
    L = efla.lib()
    nul, fake = None, 4096
    need = efla.efla_chunk_bwd_workspace_size(1, 1, 64, 16, 16, 16, torch.float32)
    assert need > efla.efla_chunk_fwd_workspace_size(1, 1, 64, 16, 16, 16, torch.float32)

    def fwd(B=1, L_=64, dk=16, C=16, rule=0, p=fake, ws=nul, wsb=0, sf=nul):
        return L.efla_chunk_fwd_train(p, p, p, p, nul, p, sf, B, 1, L_, dk, 16, C, 0, rule, ws, wsb, nul)

    assert fwd(rule=3) == 1 and fwd(B=0) == 1 and fwd(dk=24) == 2 and fwd(C=48) == 2
    assert fwd(p=nul) == 1 and fwd(p=fake + 4) == 1
    assert fwd() == 3 and fwd(ws=fake, wsb=need - 1) == 3  # the forward's own size is too small
    assert fwd(L_=0, p=nul) == 0                          # nothing to do, no final state wanted

    def bwd(B=1, L_=64, dk=16, C=16, rule=0, p=fake, ws=nul, wsb=0, ds0=nul):
        return L.efla_chunk_bwd_train(p, p, p, p, nul, p, nul, p, p, p, p, ds0, B, 1, L_, dk, 16, C, 0, rule, ws,
                                      wsb, nul)

    assert bwd(rule=3) == 1 and bwd(B=0) == 1 and bwd(dk=24) == 2 and bwd(C=48) == 2
    assert bwd(p=nul) == 1 and bwd(p=fake + 4) == 1
    assert bwd() == 3 and bwd(ws=fake, wsb=need - 1) == 3
    assert bwd(L_=0, p=nul) == 0


def test_segmented_workspace_size_and_validation():
    f = efla.efla_chunk_fwd_segmented_workspace_size
    assert f(1, 1, 0, 16, 16, 16, 4, torch.float32) == 0
    assert f(1, 1, 64, 16, 16, 16, 0, torch.float32) == 0
    # stiff_64k with 4 segments: T slots, offsets, M, N and incoming states
    U, slots = 4, 16 * (65536 // 64 + 4)
    r = lambda x: (x + 255) // 256 * 256
    want = r(slots * 64 * 64 * 2) + r((U + 1) * 4) + r(U * 16 * 128 * 128 * 4) + 2 * r(U * 16 * 128 * 128 * 4)
    assert f(1, 16, 65536, 128, 128, 64, 4, torch.bfloat16) == want
    assert efla.default_segments(1, 16, 65536, 128, 64) == 4
    assert efla.default_segments(4, 16, 4096, 128, 64) == 1
    assert efla.default_segments(1, 1, 64, 128, 64) == 1
    L = efla.lib()
    nul, fake = None, 4096

    def call(seg=4, rule=0, p=fake, ws=nul, wsb=0, L_=256):
        return L.efla_chunk_fwd_segmented(p, p, p, p, nul, p, nul, 1, 1, L_, 16, 16, 16, seg, 0, rule, ws, wsb, nul)

    assert call(seg=0) == 1 and call(rule=5) == 1 and call(p=nul) == 1 and call(p=fake + 8) == 1
    assert call() == 3 and call(ws=fake, wsb=64) == 3


def test_noalloc_rejects_problems_beyond_its_scratch():
    """efla_chunk_fwd_noalloc checks the size against its fixed scratch before
    any HIP call (so this runs without a GPU)."""
    L = efla.lib()
    nul, fake = None, ctypes.c_void_p(4096)
    # 4 x 16 x 4096 tokens in chunks of 64, bf16: 32 MiB of T -> fits; 3x the batch -> 96 MiB does not
    need = efla.efla_chunk_fwd_workspace_size(12, 16, 4096, 128, 128, 64, torch.bfloat16)
    assert need > efla.NOALLOC_SCRATCH_BYTES
    assert L.efla_chunk_fwd_noalloc(fake, fake, fake, fake, nul, fake, nul, 12, 16, 4096, 128, 128, 64, 1, 0,
                                    nul) == 5
    assert efla.efla_chunk_fwd_workspace_size(4, 16, 4096, 128, 128, 64, torch.bfloat16) <= efla.NOALLOC_SCRATCH_BYTES
    # ordinary validation first: unsupported sizes, bad rule
    assert L.efla_chunk_fwd_noalloc(nul, nul, nul, nul, nul, nul, nul, 1, 1, 64, 24, 16, 16, 0, 0, nul) == 2
    assert L.efla_chunk_fwd_noalloc(nul, nul, nul, nul, nul, nul, nul, 1, 1, 64, 16, 16, 16, 0, 7, nul) == 1
    # nothing to do is success without a launch
    assert L.efla_chunk_fwd_noalloc(nul, nul, nul, nul, nul, nul, nul, 1, 1, 0, 16, 16, 16, 0, 0, nul) == 0
