"""Python binding of libaa.so, the MI355X row-typed associative-algebra projection.

The functions carry the names of the C entry points in include/aa.h and only
marshal arguments: torch tensors are passed as device pointers (data_ptr) and
the current torch stream as the HIP stream.  Every step of the computation
runs in the library's HIP kernels; there is no fallback.  Loading fails
loudly when libaa.so has not been built.

Build first:  python -m associative_algebra_block_amd.build
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded before libaa.so so that both share torch's HIP runtime

__all__ = [
    "AA_LAW_QQ", "AA_LAW_Q2XQ2", "AA_LAW_DIGRAPH", "AA_TYPES_POS_MOD", "AA_TYPES_BLOCK_ROWS", "AA_TYPES_EXPLICIT",
    "AA_BF16", "AA_F32", "AA_OK", "AA_ERR_INVALID_ARG", "AA_ERR_SHAPE", "AA_ERR_UNSUPPORTED",
    "AA_ERR_HIP", "AAError", "Plan", "lib_path", "load",
    "aa_plan_create", "aa_plan_create_digraph", "aa_plan_destroy", "aa_plan_info", "aa_packed_layout_version",
    "aa_pack_weights", "aa_unpack_weights",
    "aa_project_fwd", "aa_swiglu_ffn_fwd", "aa_swiglu_ffn_fwd_noalloc", "aa_decode_gemv", "aa_project_bwd_workspace",
    "aa_project_bwd_data", "aa_project_bwd_weight", "aa_set_kernel_events", "aa_status_string", "aa_last_error",
]

AA_LAW_QQ, AA_LAW_Q2XQ2, AA_LAW_DIGRAPH = 0, 1, 2
AA_TYPES_POS_MOD, AA_TYPES_BLOCK_ROWS, AA_TYPES_EXPLICIT = 0, 1, 2
AA_BF16, AA_F32 = 0, 1
AA_OK, AA_ERR_INVALID_ARG, AA_ERR_SHAPE, AA_ERR_UNSUPPORTED, AA_ERR_HIP = 0, 1, 2, 3, 4

_LAWS = {"Qq": AA_LAW_QQ, "Q2xQ2": AA_LAW_Q2XQ2, "digraph": AA_LAW_DIGRAPH, AA_LAW_QQ: AA_LAW_QQ,
         AA_LAW_Q2XQ2: AA_LAW_Q2XQ2, AA_LAW_DIGRAPH: AA_LAW_DIGRAPH}
_KINDS = {"pos_mod": AA_TYPES_POS_MOD, "block_rows": AA_TYPES_BLOCK_ROWS, "explicit": AA_TYPES_EXPLICIT,
          AA_TYPES_POS_MOD: AA_TYPES_POS_MOD, AA_TYPES_BLOCK_ROWS: AA_TYPES_BLOCK_ROWS,
          AA_TYPES_EXPLICIT: AA_TYPES_EXPLICIT}
_DTYPES = {"bf16": AA_BF16, "f32": AA_F32, torch.bfloat16: AA_BF16, torch.float32: AA_F32,
           AA_BF16: AA_BF16, AA_F32: AA_F32}
_TORCH_DTYPE = {AA_BF16: torch.bfloat16, AA_F32: torch.float32}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_c_i32, _c_i64, _c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
_SIGNATURES = {
    "aa_plan_create": (ctypes.c_int, [ctypes.POINTER(_c_p), ctypes.c_int, _c_i32, _c_i64, _c_i64, ctypes.c_int,
                                      _c_i64, ctypes.c_int, ctypes.c_int]),
    "aa_plan_create_digraph": (ctypes.c_int, [ctypes.POINTER(_c_p), _c_i32, ctypes.c_char_p, _c_i64, _c_i64,
                                              ctypes.c_int, _c_i64, ctypes.c_int, ctypes.c_int]),
    "aa_plan_destroy": (ctypes.c_int, [_c_p]),
    "aa_plan_info": (ctypes.c_int, [_c_p, ctypes.POINTER(_c_i64), ctypes.POINTER(_c_i64), ctypes.POINTER(_c_i64)]),
    "aa_packed_layout_version": (ctypes.c_int, [_c_p, ctypes.POINTER(_c_i32)]),
    "aa_pack_weights": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p]),
    "aa_unpack_weights": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p]),
    "aa_project_fwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p]),
    "aa_swiglu_ffn_fwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_p,
                                         _c_p]),
    "aa_swiglu_ffn_fwd_noalloc": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64,
                                                 _c_p, _c_p]),
    "aa_decode_gemv": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p]),
    "aa_project_bwd_workspace": (ctypes.c_int, [_c_p, _c_i64, ctypes.POINTER(ctypes.c_size_t),
                                                ctypes.POINTER(ctypes.c_size_t)]),
    "aa_project_bwd_data": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, ctypes.c_size_t,
                                           _c_p]),
    "aa_project_bwd_weight": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, ctypes.c_size_t,
                                             _c_p]),
    "aa_set_kernel_events": (ctypes.c_int, [_c_p, _c_p]),
    "aa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "aa_last_error": (ctypes.c_char_p, []),
}
EXPORTED = tuple(_SIGNATURES)


def lib_path() -> str:
    return os.path.join(_HERE, "libaa.so")


def load():
    """Load libaa.so (once) and declare its signatures.  Raises if it is missing."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run `python -m associative_algebra_block_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


class AAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {aa_status_string(status)}: {detail}")


def _check(status: int, where: str):
    if status != AA_OK:
        raise AAError(status, where, aa_last_error())


def aa_status_string(status: int) -> str:
    return load().aa_status_string(int(status)).decode()


def aa_last_error() -> str:
    return load().aa_last_error().decode()


class Plan:
    """An aa_plan_t with the arguments it was created from."""

    def __init__(self, handle, law, q, d_in, d_out, type_kind, period, in_dtype, out_dtype):
        self.handle = handle
        self.law, self.q, self.d_in, self.d_out = law, q, d_in, d_out
        self.type_kind, self.period = type_kind, period
        self.in_dtype, self.out_dtype = in_dtype, out_dtype

    @property
    def b_in(self):
        return self.d_in // self.q

    @property
    def b_out(self):
        return self.d_out // self.q

    @property
    def in_torch_dtype(self):
        return _TORCH_DTYPE[self.in_dtype]

    @property
    def out_torch_dtype(self):
        return _TORCH_DTYPE[self.out_dtype]

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.aa_plan_destroy(self.handle)
            self.handle = None


def _ptr(t, name, dtype=None, numel=None):
    """Device pointer of a tensor (or an int address / None passed through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def aa_plan_create(law, q, d_in, d_out, type_kind="pos_mod", period=0, in_dtype="bf16", out_dtype="bf16") -> Plan:
    lib = load()
    h = _c_p()
    law_, kind_, din_, dout_ = _LAWS[law], _KINDS[type_kind], _DTYPES[in_dtype], _DTYPES[out_dtype]
    _check(lib.aa_plan_create(ctypes.byref(h), law_, int(q), int(d_in), int(d_out), kind_, int(period), din_,
                              dout_), "aa_plan_create")
    return Plan(h.value, law_, int(q), int(d_in), int(d_out), kind_, int(period), din_, dout_)


def aa_plan_create_digraph(q, edges, d_in, d_out, type_kind="pos_mod", period=0, in_dtype="bf16",
                           out_dtype="bf16") -> Plan:
    """Plan for the table of a directed graph on q groups; `edges` is an
    iterable of (i, k) pairs (i -> k) or a q x q 0/1 array."""
    lib = load()
    q = int(q)
    adj = bytearray(q * q)
    if hasattr(edges, "shape"):
        for i in range(q):
            for k in range(q):
                adj[i * q + k] = 1 if edges[i][k] else 0
    else:
        for i, k in edges:
            adj[int(i) * q + int(k)] = 1
    h = _c_p()
    kind_, din_, dout_ = _KINDS[type_kind], _DTYPES[in_dtype], _DTYPES[out_dtype]
    _check(lib.aa_plan_create_digraph(ctypes.byref(h), q, bytes(adj), int(d_in), int(d_out), kind_, int(period),
                                      din_, dout_), "aa_plan_create_digraph")
    return Plan(h.value, AA_LAW_DIGRAPH, q, int(d_in), int(d_out), kind_, int(period), din_, dout_)


def aa_plan_destroy(plan: Plan):
    if plan.handle:
        _check(load().aa_plan_destroy(plan.handle), "aa_plan_destroy")
        plan.handle = None


def aa_plan_info(plan: Plan):
    a, b, c = _c_i64(), _c_i64(), _c_i64()
    _check(load().aa_plan_info(plan.handle, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "aa_plan_info")
    return a.value, b.value, c.value


def aa_packed_layout_version(plan: Plan) -> int:
    v = _c_i32()
    _check(load().aa_packed_layout_version(plan.handle, ctypes.byref(v)), "aa_packed_layout_version")
    return int(v.value)


def aa_pack_weights(plan: Plan, W_rowmajor, W_packed, stream=None):
    n = plan.d_in * plan.d_out
    _check(load().aa_pack_weights(plan.handle, _ptr(W_rowmajor, "W_rowmajor", plan.in_torch_dtype, n),
                                  _ptr(W_packed, "W_packed", plan.in_torch_dtype, n), _stream(stream)),
           "aa_pack_weights")


def aa_unpack_weights(plan: Plan, W_packed, W_rowmajor, stream=None):
    n = plan.d_in * plan.d_out
    _check(load().aa_unpack_weights(plan.handle, _ptr(W_packed, "W_packed", plan.in_torch_dtype, n),
                                    _ptr(W_rowmajor, "W_rowmajor", plan.in_torch_dtype, n), _stream(stream)),
           "aa_unpack_weights")


def _rows_of(t, M):
    if M is not None:
        return int(M)
    return int(t.shape[0])


def aa_project_fwd(plan: Plan, X, W_packed, Y, M=None, pos_offset=0, row_types=None, stream=None):
    M = _rows_of(X, M)
    _check(load().aa_project_fwd(
        plan.handle, _ptr(X, "X", plan.in_torch_dtype, M * plan.d_in),
        _ptr(W_packed, "W_packed", plan.in_torch_dtype, plan.d_in * plan.d_out),
        _ptr(Y, "Y", plan.out_torch_dtype, M * plan.d_out), M, int(pos_offset),
        _ptr(row_types, "row_types", torch.int32, M), _stream(stream)), "aa_project_fwd")


def aa_swiglu_ffn_fwd(up: Plan, down: Plan, X, Wg_packed, Wu_packed, Wd_packed, H, Y, M=None, pos_offset=0,
                      row_types=None, stream=None):
    M = _rows_of(X, M)
    nw = up.d_in * up.d_out
    _check(load().aa_swiglu_ffn_fwd(
        up.handle, down.handle, _ptr(X, "X", up.in_torch_dtype, M * up.d_in),
        _ptr(Wg_packed, "Wg_packed", up.in_torch_dtype, nw), _ptr(Wu_packed, "Wu_packed", up.in_torch_dtype, nw),
        _ptr(Wd_packed, "Wd_packed", down.in_torch_dtype, down.d_in * down.d_out),
        _ptr(H, "H", up.out_torch_dtype, M * up.d_out), _ptr(Y, "Y", down.out_torch_dtype, M * down.d_out),
        M, int(pos_offset), _ptr(row_types, "row_types", torch.int32, M), _stream(stream)), "aa_swiglu_ffn_fwd")


def aa_swiglu_ffn_fwd_noalloc(up: Plan, down: Plan, X, Wg_packed, Wu_packed, Wd_packed, Y, M=None, pos_offset=0,
                              row_types=None, stream=None):
    """aa_swiglu_ffn_fwd with the hidden activation in the library's static
    device scratch (no H argument; at most AA_NOALLOC_SCRATCH_BYTES of it)."""
    M = _rows_of(X, M)
    nw = up.d_in * up.d_out
    _check(load().aa_swiglu_ffn_fwd_noalloc(
        up.handle, down.handle, _ptr(X, "X", up.in_torch_dtype, M * up.d_in),
        _ptr(Wg_packed, "Wg_packed", up.in_torch_dtype, nw), _ptr(Wu_packed, "Wu_packed", up.in_torch_dtype, nw),
        _ptr(Wd_packed, "Wd_packed", down.in_torch_dtype, down.d_in * down.d_out),
        _ptr(Y, "Y", down.out_torch_dtype, M * down.d_out), M, int(pos_offset),
        _ptr(row_types, "row_types", torch.int32, M), _stream(stream)), "aa_swiglu_ffn_fwd_noalloc")


AA_NOALLOC_SCRATCH_BYTES = 64 << 20


def aa_decode_gemv(plan: Plan, x, W_packed, y, n=None, pos_offset=0, row_types=None, stream=None):
    n = _rows_of(x, n)
    _check(load().aa_decode_gemv(
        plan.handle, _ptr(x, "x", plan.in_torch_dtype, n * plan.d_in),
        _ptr(W_packed, "W_packed", plan.in_torch_dtype, plan.d_in * plan.d_out),
        _ptr(y, "y", plan.out_torch_dtype, n * plan.d_out), n, int(pos_offset),
        _ptr(row_types, "row_types", torch.int32, n), _stream(stream)), "aa_decode_gemv")


def aa_project_bwd_workspace(plan: Plan, M: int) -> tuple[int, int]:
    """(bytes for aa_project_bwd_data, bytes for aa_project_bwd_weight)."""
    nd, nw = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(load().aa_project_bwd_workspace(plan.handle, int(M), ctypes.byref(nd), ctypes.byref(nw)),
           "aa_project_bwd_workspace")
    return int(nd.value), int(nw.value)


def aa_project_bwd_data(plan: Plan, dY, W_packed, dX, M=None, pos_offset=0, row_types=None, workspace=None,
                        workspace_bytes=None, stream=None):
    M = _rows_of(dY, M)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().aa_project_bwd_data(
        plan.handle, _ptr(dY, "dY", plan.in_torch_dtype, M * plan.d_out),
        _ptr(W_packed, "W_packed", plan.in_torch_dtype, plan.d_in * plan.d_out),
        _ptr(dX, "dX", plan.out_torch_dtype, M * plan.d_in), M, int(pos_offset),
        _ptr(row_types, "row_types", torch.int32, M), _ptr(workspace, "workspace"), int(workspace_bytes),
        _stream(stream)), "aa_project_bwd_data")


def aa_project_bwd_weight(plan: Plan, X, dY, dW_packed, M=None, pos_offset=0, row_types=None, workspace=None,
                          workspace_bytes=None, stream=None):
    M = _rows_of(X, M)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().aa_project_bwd_weight(
        plan.handle, _ptr(X, "X", plan.in_torch_dtype, M * plan.d_in),
        _ptr(dY, "dY", plan.in_torch_dtype, M * plan.d_out),
        _ptr(dW_packed, "dW_packed", plan.out_torch_dtype, plan.d_in * plan.d_out), M, int(pos_offset),
        _ptr(row_types, "row_types", torch.int32, M), _ptr(workspace, "workspace"), int(workspace_bytes),
        _stream(stream)), "aa_project_bwd_weight")


def _event(ev):
    if ev is None:
        return None
    if isinstance(ev, torch.cuda.Event):
        h = ev.cuda_event
        if not h:
            raise ValueError("aa_set_kernel_events: a torch.cuda.Event exists only after its first record()")
        return h
    return int(ev)


def aa_set_kernel_events(start=None, stop=None):
    """Hand the next kernel launched from this thread the start event and every
    later one the stop event (torch.cuda.Event with timing, or raw handles);
    (None, None) switches this off."""
    _check(load().aa_set_kernel_events(_event(start), _event(stop)), "aa_set_kernel_events")


# ----------------------------------------------------------- conveniences ---

def pack(plan: Plan, W: torch.Tensor, stream=None) -> torch.Tensor:
    """Return a new block-packed copy of the row-major weight W."""
    out = torch.empty(plan.d_in * plan.d_out, dtype=plan.in_torch_dtype, device=W.device)
    aa_pack_weights(plan, W, out, stream)
    return out


def project(plan: Plan, X, W_packed, pos_offset=0, row_types=None, stream=None) -> torch.Tensor:
    Y = torch.empty(X.shape[0], plan.d_out, dtype=plan.out_torch_dtype, device=X.device)
    aa_project_fwd(plan, X, W_packed, Y, None, pos_offset, row_types, stream)
    return Y
