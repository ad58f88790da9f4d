"""ctypes binding of libfa2.so -- argument marshalling only.

Every step of the forward and backward passes runs in the HIP library.  There is no fallback:
if libfa2.so is missing or fails to load, every entry point raises.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa2.so")

FA2_OK = 0
STATUS_NAMES = {
    0: "FA2_OK", 1: "FA2_ERR_NULL", 2: "FA2_ERR_DIM", 3: "FA2_ERR_UNSUPPORTED_D",
    4: "FA2_ERR_ARG", 5: "FA2_ERR_ALIGN", 6: "FA2_ERR_DEVICE", 7: "FA2_ERR_LAUNCH",
    8: "FA2_ERR_WORKSPACE", 9: "FA2_ERR_SCRATCH",
}
FA2_MAX_SPLITS = 128
FA2_STATIC_SCRATCH_BYTES = 32 * 1024 * 1024

# name -> (restype, argtypes), exactly the declarations of include/fa2.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
_L = ctypes.c_int64
_D = ctypes.c_double
_U64 = ctypes.c_uint64
_U32 = ctypes.c_uint32
SIGNATURES = {
    "fa2_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa2_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa2_fwd_f16": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa2_status_string": (ctypes.c_char_p, [_I]),
    "fa2_check_args": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I]),
    "fa2_fwd_splitkv": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _P]),
    "fa2_fwd_splitkv_static": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa2_splitkv_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "fa2_splitkv_num_splits": (_I, [_I, _I, _I, _I, _I, _I]),
    "fa2_merge_partials": (_I, [_P, _P, _I, _L, _I, _P, _P, _P]),
    "fa2_fwd_window": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa2_fwd_dropout": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _D, _U64, _U32, _P]),
    "fa2_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]),
    "fa2_bwd_workspace_bytes": (_Z, [_I, _I, _I]),
    "fa2_bwd_f16": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]),
    "fa2_bwd_window": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _P]),
    "fa2_bwd_dropout": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _D, _U64, _U32, _P, _Z,
                             _P]),
}
# fp16 twins: the same arguments
for _n in ("fa2_fwd_window", "fa2_fwd_dropout", "fa2_fwd_splitkv", "fa2_merge_partials", "fa2_bwd_window",
           "fa2_bwd_dropout"):
    SIGNATURES[_n + "_f16"] = SIGNATURES[_n]

_lib = None


class FA2Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, status_string(status), STATUS_NAMES.get(status, status)))


def lib():
    """The loaded libfa2.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libfa2.so is not built (%s); build it with "
                "`python -m flashattention_forward_fwd_amd.build` or __graft_entry__.build()" % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status):
    return lib().fa2_status_string(int(status)).decode()


def _arg(x):
    """A tensor becomes its device address (data_ptr); everything else passes as is
    (ctypes converts it by the declared argument type)."""
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return x


def _call(name, *args):
    """Call the libfa2 entry point `name`; raise FA2Error on a non-OK status."""
    st = getattr(lib(), name)(*(_arg(a) for a in args))
    if st != FA2_OK:
        raise FA2Error(st, name)


# Entry points that return an fa2_status: tensors or raw device addresses; raise FA2Error.
def fa2_fwd(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, stream):
    """``fa2_fwd`` (bf16)."""
    _call("fa2_fwd", q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, stream)


def fa2_fwd_f16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, stream):
    """``fa2_fwd_f16`` (fp16)."""
    _call("fa2_fwd_f16", q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, stream)


def fa2_fwd_f32(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, stream):
    """``fa2_fwd_f32`` (fp32)."""
    _call("fa2_fwd_f32", q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, stream)


def fa2_fwd_window(q, k, v, o, lse, B, H, Lq, Lk, d, scale, window_left, window_right, stream):
    """``fa2_fwd_window`` (bf16, keys i - window_left .. i + window_right)."""
    _call("fa2_fwd_window", q, k, v, o, lse, B, H, Lq, Lk, d, scale, window_left, window_right, stream)


def fa2_fwd_window_f16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, window_left, window_right, stream):
    """``fa2_fwd_window_f16`` (fp16)."""
    _call("fa2_fwd_window_f16", q, k, v, o, lse, B, H, Lq, Lk, d, scale, window_left, window_right, stream)


def fa2_fwd_dropout(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, dropout_p, seed, offset, stream):
    """``fa2_fwd_dropout`` (bf16, Philox keep mask of (seed, offset))."""
    _call("fa2_fwd_dropout", q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, dropout_p, seed, offset, stream)


def fa2_fwd_dropout_f16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, dropout_p, seed, offset, stream):
    """``fa2_fwd_dropout_f16`` (fp16)."""
    _call("fa2_fwd_dropout_f16", q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, dropout_p, seed, offset,
          stream)


def fa2_fwd_splitkv(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, num_splits, workspace, workspace_bytes,
                    stream):
    """``fa2_fwd_splitkv`` (bf16, split K/V + merge)."""
    _call("fa2_fwd_splitkv", q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, num_splits, workspace,
          workspace_bytes, stream)


def fa2_fwd_splitkv_f16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, num_splits, workspace,
                        workspace_bytes, stream):
    """``fa2_fwd_splitkv_f16`` (fp16)."""
    _call("fa2_fwd_splitkv_f16", q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, num_splits, workspace,
          workspace_bytes, stream)


def fa2_fwd_splitkv_static(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, num_splits, stream):
    """``fa2_fwd_splitkv_static`` (bf16 split K/V + merge, partials in the library's static scratch)."""
    _call("fa2_fwd_splitkv_static", q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, num_splits, stream)


def fa2_merge_partials(o_parts, lse_parts, n_parts, rows, d, o, lse, stream):
    """``fa2_merge_partials`` (bf16 output)."""
    _call("fa2_merge_partials", o_parts, lse_parts, n_parts, rows, d, o, lse, stream)


def fa2_merge_partials_f16(o_parts, lse_parts, n_parts, rows, d, o, lse, stream):
    """``fa2_merge_partials_f16`` (fp16 output)."""
    _call("fa2_merge_partials_f16", o_parts, lse_parts, n_parts, rows, d, o, lse, stream)


def fa2_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, workspace, workspace_bytes,
            stream):
    """``fa2_bwd`` (bf16 gradients dq, dk, dv)."""
    _call("fa2_bwd", q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, workspace,
          workspace_bytes, stream)


def fa2_bwd_f16(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, workspace, workspace_bytes,
                stream):
    """``fa2_bwd_f16`` (fp16 gradients)."""
    _call("fa2_bwd_f16", q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, workspace,
          workspace_bytes, stream)


def fa2_bwd_window(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, window_left, window_right,
                   workspace, workspace_bytes, stream):
    """``fa2_bwd_window`` (gradients of fa2_fwd_window)."""
    _call("fa2_bwd_window", q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, window_left,
          window_right, workspace, workspace_bytes, stream)


def fa2_bwd_window_f16(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, window_left, window_right,
                       workspace, workspace_bytes, stream):
    """``fa2_bwd_window_f16`` (gradients of fa2_fwd_window_f16)."""
    _call("fa2_bwd_window_f16", q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, window_left,
          window_right, workspace, workspace_bytes, stream)


def fa2_bwd_dropout(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, dropout_p, seed, offset,
                    workspace, workspace_bytes, stream):
    """``fa2_bwd_dropout`` (gradients of fa2_fwd_dropout)."""
    _call("fa2_bwd_dropout", q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, dropout_p, seed,
          offset, workspace, workspace_bytes, stream)


def fa2_bwd_dropout_f16(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, dropout_p, seed,
                        offset, workspace, workspace_bytes, stream):
    """``fa2_bwd_dropout_f16`` (gradients of fa2_fwd_dropout_f16)."""
    _call("fa2_bwd_dropout_f16", q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, dropout_p,
          seed, offset, workspace, workspace_bytes, stream)


# Size and query helpers (no status).
def fa2_check_args(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, elem_bytes):
    """``fa2_check_args``: the status the entry points would return (no HIP call)."""
    return lib().fa2_check_args(*(_arg(a) for a in (q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, elem_bytes)))


def fa2_splitkv_workspace_bytes(B, H, Lq, Lk, d, causal, num_splits):
    """``fa2_splitkv_workspace_bytes``: bytes of workspace (0: sizes rejected)."""
    return lib().fa2_splitkv_workspace_bytes(B, H, Lq, Lk, d, causal, num_splits)


def fa2_splitkv_num_splits(B, H, Lq, Lk, d, causal):
    """``fa2_splitkv_num_splits``: the split count that num_splits=0 selects."""
    return lib().fa2_splitkv_num_splits(B, H, Lq, Lk, d, causal)


def fa2_bwd_workspace_bytes(B, H, Lq):
    """``fa2_bwd_workspace_bytes``: bytes of backward workspace (0: sizes rejected)."""
    return lib().fa2_bwd_workspace_bytes(B, H, Lq)
