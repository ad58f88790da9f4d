"""C-ABI checks that need no GPU: the library loads, exports every function that
include/fa2.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import flashattention_forward_fwd_amd as fa
from flashattention_forward_fwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert header_functions() == sorted(["fa2_fwd", "fa2_fwd_f16", "fa2_fwd_f32", "fa2_status_string", "fa2_check_args",
                                         "fa2_fwd_splitkv", "fa2_splitkv_workspace_bytes",
                                         "fa2_splitkv_num_splits", "fa2_merge_partials",
                                         "fa2_bwd", "fa2_bwd_workspace_bytes", "fa2_fwd_window",
                                         "fa2_bwd_window", "fa2_bwd_f16", "fa2_fwd_dropout",
                                         "fa2_bwd_dropout", "fa2_fwd_window_f16", "fa2_fwd_dropout_f16",
                                         "fa2_fwd_splitkv_f16", "fa2_merge_partials_f16",
                                         "fa2_bwd_window_f16", "fa2_bwd_dropout_f16", "fa2_fwd_splitkv_static"])


PAGE_TITLES = ("Flash Attention 全解析", "FlashAttention 怎么做", "Triton内核实战",
               "FlashAttention-2 算法架构升级", "新年一定要学会FlashAttention")


def declaration_comments():
    """(name, comment block just before the declaration) for every function in the header."""
    text = open(HEADER).read()
    pat = r"(/\*(?:(?!\*/).)*\*/)\s*(?:#define[^\n]*\n\s*)*(?:int|size_t|const char \*)\s*(fa2_\w+)\s*\("
    out = []
    for m in re.finditer(pat, text, flags=re.S):
        body = re.sub(r"\s*\n\s*\*\s*", " ", m.group(1))      # join comment lines
        out.append((m.group(2), body))
    return out


def test_every_declaration_cites_a_page():
    """Each entry point's comment names the page (by title) that defines what it
    computes; the no-allocation variant names the callers it is for instead."""
    blocks = dict(declaration_comments())
    assert sorted(blocks) == header_functions()
    for name, body in blocks.items():
        if name == "fa2_fwd_splitkv_static":
            assert "cannot allocate" in body
            continue
        assert any(t in body for t in PAGE_TITLES), name


def test_f16_twins_reject_like_their_bf16_entry_points():
    L = fa.lib()
    big = 1 << 30
    assert L.fa2_fwd_window_f16(None, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 4, 0, None) == 1
    assert L.fa2_fwd_window_f16(A, A, A, A, A, 1, 1, 8, 8, 80, 0.1, 4, 0, None) == 3
    assert L.fa2_fwd_dropout_f16(A, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 1, 1.0, 1, 0, None) == 4
    assert L.fa2_fwd_splitkv_f16(A, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 0, -1, A, big, None) == 4
    assert L.fa2_merge_partials_f16(A, A, 0, 10, 64, A, A, None) == 4
    assert L.fa2_bwd_window_f16(*([A] * 9), 1, 1, 8, 8, 64, 0.1, 4, 0, A, 4, None) == 8
    assert L.fa2_bwd_dropout_f16(*([A] * 9), 1, 1, 8, 8, 64, 0.1, 1, -0.5, 1, 0, A, big, None) == 4


def test_library_exports_every_declared_symbol():
    handle = ctypes.CDLL(_lib.LIB_PATH)
    for name in header_functions():
        assert hasattr(handle, name), name
    assert set(header_functions()) == set(_lib.SIGNATURES)


def test_status_strings():
    for code in range(10):
        assert fa.status_string(code) != "unknown status"
    assert fa.status_string(99) == "unknown status"


A = 1 << 20   # a 16-byte-aligned fake address (never dereferenced: checks run first)


@pytest.mark.parametrize("elem", [2, 4])
def test_argument_checks(elem):
    ok = dict(q=A, k=A, v=A, o=A, lse=A, B=2, H=3, Lq=100, Lk=77, d=128, scale=0.1, causal=1)

    def st(**kw):
        a = dict(ok, **kw)
        return fa.fa2_check_args(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Lq"],
                                 a["Lk"], a["d"], a["scale"], a["causal"], elem)
    assert st() == 0
    assert st(d=64) == 0 and st(d=32) == 0 and st(d=128) == 0
    assert st(q=0) == 1 and st(lse=0) == 1 and st(v=0) == 1
    assert st(B=0) == 2 and st(H=-1) == 2 and st(Lq=0) == 2 and st(Lk=0) == 2
    assert st(B=1 << 30, H=1 << 30) == 2
    for d in (0, 16, 80, 112, 512, 127):
        assert st(d=d) == 3
    assert st(d=256) == (0 if elem == 2 else 3)      # d = 96, 256: 16-bit data only
    assert st(d=96) == (0 if elem == 2 else 3)
    assert st(causal=2) == 4 and st(causal=-1) == 4
    assert st(scale=0.0) == 4 and st(scale=-1.0) == 4
    assert st(scale=float("inf")) == 4 and st(scale=float("nan")) == 4
    assert st(q=A + 2) == 5 and st(o=A + 8) == 5 and st(lse=A + 4) == 5


def test_entry_points_reject_before_touching_the_device():
    """fa2_fwd / fa2_fwd_f32 return the validation status without any HIP call."""
    L = fa.lib()
    for fn in (L.fa2_fwd, L.fa2_fwd_f32):
        assert fn(None, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 0, None) == 1
        assert fn(A, A, A, A, A, 1, 1, 8, 8, 80, 0.1, 0, None) == 3
        assert fn(A, A, A, A, A, 1, 0, 8, 8, 64, 0.1, 0, None) == 2
        assert fn(A, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 3, None) == 4
        assert fn(A, A + 6, A, A, A, 1, 1, 8, 8, 64, 0.1, 0, None) == 5


def test_binding_raises_on_error_status():
    with pytest.raises(fa.FA2Error) as e:
        fa.fa2_fwd(A, A, A, A, A, 1, 1, 8, 8, 80, 0.1, 0, None)
    assert e.value.status == 3


def test_forward_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


def test_splitkv_rejects_before_touching_the_device():
    """Bad sizes, split counts and workspaces are refused before any HIP call."""
    L = fa.lib()
    f = L.fa2_fwd_splitkv
    big = 1 << 30
    assert f(None, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 0, 1, A, big, None) == 1
    assert f(A, A, A, A, A, 1, 1, 8, 8, 80, 0.1, 0, 1, A, big, None) == 3
    assert f(A, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 0, -1, A, big, None) == 4
    assert f(A, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 0, fa.FA2_MAX_SPLITS + 1, A, big, None) == 4
    assert f(A, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 0, 2, None, big, None) == 8
    assert f(A, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 0, 2, A + 4, big, None) == 5


def test_splitkv_workspace_bytes():
    """Partial outputs [S, rows, d] fp32, padded to 256 bytes, then [S, rows] fp32."""
    for (B, H, Lq, d, S) in [(1, 1, 1, 64, 1), (2, 3, 100, 128, 4), (1, 2, 77, 64, 3)]:
        rows = B * H * Lq
        o_bytes = -(-S * rows * d * 4 // 256) * 256
        assert fa.fa2_splitkv_workspace_bytes(B, H, Lq, 500, d, 0, S) == o_bytes + S * rows * 4
    assert fa.fa2_splitkv_workspace_bytes(1, 1, 8, 8, 80, 0, 2) == 0
    assert fa.fa2_splitkv_workspace_bytes(1, 1, 8, 8, 96, 0, 2) > 0
    assert fa.fa2_splitkv_workspace_bytes(0, 1, 8, 8, 64, 0, 2) == 0
    assert fa.fa2_splitkv_workspace_bytes(1, 1, 8, 8, 64, 0, fa.FA2_MAX_SPLITS + 1) == 0


def test_head_size_limit():
    """One head's K must stay below 2 GiB (32-bit tile offsets)."""
    # (Lk + 64) * d * element size <= 2^31 - 1
    assert fa.fa2_check_args(A, A, A, A, A, 1, 1, 8, (1 << 23) - 65, 128, 0.1, 0, 2) == 0
    assert fa.fa2_check_args(A, A, A, A, A, 1, 1, 8, (1 << 23) - 64, 128, 0.1, 0, 2) == 2
    assert fa.fa2_check_args(A, A, A, A, A, 1, 1, 8, (1 << 23) - 65, 64, 0.1, 0, 4) == 0
    assert fa.fa2_check_args(A, A, A, A, A, 1, 1, 8, (1 << 23) - 64, 64, 0.1, 0, 4) == 2


def test_merge_rejects_before_touching_the_device():
    f = fa.lib().fa2_merge_partials
    assert f(None, A, 2, 10, 64, A, A, None) == 1
    assert f(A, A, 0, 10, 64, A, A, None) == 4
    assert f(A, A, fa.FA2_MAX_SPLITS + 1, 10, 64, A, A, None) == 4
    assert f(A, A, 2, 0, 64, A, A, None) == 2
    assert f(A, A, 2, 10, 80, A, A, None) == 3
    assert f(A, A + 4, 2, 10, 64, A, A, None) == 5


def test_bwd_rejects_before_touching_the_device():
    """fa2_bwd refuses bad pointers, sizes and workspaces before any HIP call."""
    f = fa.lib().fa2_bwd
    big = 1 << 30
    args = lambda **kw: [kw.get(n, A) for n in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv")]
    assert f(*args(do=None), 1, 1, 8, 8, 64, 0.1, 0, A, big, None) == 1
    assert f(*args(dk=None), 1, 1, 8, 8, 64, 0.1, 0, A, big, None) == 1
    assert f(*args(q=None), 1, 1, 8, 8, 64, 0.1, 0, A, big, None) == 1
    assert f(*args(), 1, 1, 8, 8, 80, 0.1, 0, A, big, None) == 3
    assert f(*args(), 1, 1, 8, 8, 512, 0.1, 0, A, big, None) == 3
    assert f(*args(), 1, 1, 0, 8, 64, 0.1, 0, A, big, None) == 2
    assert f(*args(), 1, 1, 8, 8, 64, 0.1, 2, A, big, None) == 4
    assert f(*args(dv=A + 2), 1, 1, 8, 8, 64, 0.1, 0, A, big, None) == 5
    assert f(*args(), 1, 1, 8, 8, 64, 0.1, 0, None, big, None) == 8
    assert f(*args(), 1, 1, 8, 8, 64, 0.1, 0, A + 8, big, None) == 5
    need = fa.fa2_bwd_workspace_bytes(1, 1, 8)
    assert f(*args(), 1, 1, 8, 8, 64, 0.1, 0, A, need - 1, None) == 8


def test_bwd_workspace_bytes():
    """lse * log2(e) for every query row, padded to 256 bytes, then D for every row (fp32)."""
    for (B, H, Lq) in [(1, 1, 1), (2, 3, 100), (4, 16, 2048)]:
        rows = B * H * Lq
        assert fa.fa2_bwd_workspace_bytes(B, H, Lq) == -(-rows * 4 // 256) * 256 + rows * 4
    assert fa.fa2_bwd_workspace_bytes(0, 1, 8) == 0
    assert fa.fa2_bwd_workspace_bytes(1, 1, -3) == 0


def test_backward_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 4)
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, lse, q)


def test_window_rejects_before_touching_the_device():
    f = fa.lib().fa2_fwd_window
    assert f(None, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 4, 0, None) == 1
    assert f(A, A, A, A, A, 1, 1, 8, 8, 80, 0.1, 4, 0, None) == 3
    assert f(A, A, A, A, A, 1, 1, 0, 8, 64, 0.1, 4, 0, None) == 2
    assert f(A, A, A, A, A, 1, 1, 8, 8, 64, float("nan"), 4, 0, None) == 4
    assert f(A, A, A, A, A + 4, 1, 1, 8, 8, 64, 0.1, 4, 0, None) == 5


def test_dropout_rejects_before_touching_the_device():
    f = fa.lib().fa2_fwd_dropout
    assert f(None, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 1, 0.1, 1, 0, None) == 1
    assert f(A, A, A, A, A, 1, 1, 8, 8, 80, 0.1, 1, 0.1, 1, 0, None) == 3
    assert f(A, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 2, 0.1, 1, 0, None) == 4
    for p in (-0.1, 1.0, 1.5, float("nan"), float("inf")):
        assert f(A, A, A, A, A, 1, 1, 8, 8, 64, 0.1, 1, p, 1, 0, None) == 4, p
    assert f(A, A, A, A, A + 4, 1, 1, 8, 8, 64, 0.1, 1, 0.1, 1, 0, None) == 5
    g = fa.lib().fa2_bwd_dropout
    big = 1 << 30
    assert g(None, *([A] * 8), 1, 1, 8, 8, 64, 0.1, 1, 0.1, 1, 0, A, big, None) == 1
    assert g(*([A] * 9), 1, 1, 8, 8, 80, 0.1, 1, 0.1, 1, 0, A, big, None) == 3
    assert g(*([A] * 9), 1, 1, 8, 8, 64, 0.1, 1, 1.0, 1, 0, A, big, None) == 4
    assert g(*([A] * 9), 1, 1, 8, 8, 64, 0.1, 1, 0.1, 1, 0, A, 4, None) == 8


def test_head_dims_96_and_256_only_for_16bit_data():
    # (no call here may pass every check: it would launch on the stand-in pointers)
    L = fa.lib()
    assert L.fa2_fwd_f32(A, A, A, A, A, 1, 1, 8, 8, 96, 0.1, 0, None) == 3
    assert L.fa2_fwd_f32(A, A, A, A, A, 1, 1, 8, 8, 256, 0.1, 0, None) == 3
    assert fa.fa2_splitkv_workspace_bytes(1, 1, 8, 8, 256, 0, 2) > 0
    assert fa.lib().fa2_merge_partials(A, A, 2, 10, 256, A, A + 4, None) == 5
