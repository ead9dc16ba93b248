"""Python binding of libbsa.so — causal block-sparse attention forward on MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI declared in
include/bsa.h.  The functions keep the C names; tensors are passed as device pointers (torch
is used for device memory and streams only) and a non-OK status raises BsaError.

If libbsa.so has not been built, importing this package still works but every call raises:
there is no CPU fallback.  Build it with ``python -m long_context_block_amd.build``.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbsa.so")

BSA_OK = 0
BSA_ERR_INVALID_ARGUMENT = 1
BSA_ERR_UNSUPPORTED = 2
BSA_ERR_BAD_ROUTE = 3
BSA_ERR_CAPACITY = 4
BSA_ERR_DEVICE = 5

BSA_BF16 = 0
BSA_FP32 = 1

BSA_ROUTE_BF1 = 0
BSA_ROUTE_BLOCK_DIAGONAL = 1
BSA_ROUTE_DENSE_CAUSAL = 2
BSA_ROUTE_STATIC_RANDOM = 3
BSA_ROUTE_SLIDING_WINDOW = 4

EXPORTS = ("bsa_build_route", "bsa_forward", "bsa_dense_causal_ref", "bsa_dense_route_workspace_bytes",
           "bsa_decode", "bsa_decode_routed", "bsa_decode_routed_noalloc", "bsa_decode_workspace_bytes", "bsa_build_route_transpose", "bsa_backward",
           "bsa_backward_workspace_bytes", "bsa_bsbr_forward", "bsa_bsbr_workspace_bytes", "bsa_check_route",
           "bsa_status_string", "bsa_last_error")


class BsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


class bsa_route_spec(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("n_local", ctypes.c_int32), ("keep_first", ctypes.c_int32),
                ("n_random", ctypes.c_int32), ("seed", ctypes.c_uint64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m long_context_block_amd.build`")
        # torch carries its own HIP runtime (same soname).  Load it first so that libbsa.so binds
        # to that one instance: torch's streams and device pointers are only valid there.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.bsa_build_route.argtypes = [ctypes.POINTER(bsa_route_spec), i64, i32, vp, vp, i64,
                                      ctypes.POINTER(ctypes.c_int64), vp]
        L.bsa_build_route.restype = ctypes.c_int
        L.bsa_forward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, ctypes.c_int, f32, vp, vp,
                                  i64, vp]
        L.bsa_forward.restype = ctypes.c_int
        L.bsa_dense_causal_ref.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, ctypes.c_int, f32,
                                           vp, ctypes.c_size_t, vp]
        L.bsa_dense_causal_ref.restype = ctypes.c_int
        L.bsa_dense_route_workspace_bytes.argtypes = [i64, i32]
        L.bsa_dense_route_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, ctypes.c_int, f32, vp, vp,
                                 i64, vp, ctypes.c_size_t, vp]
        L.bsa_decode.restype = ctypes.c_int
        L.bsa_decode_routed.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, ctypes.c_int, f32,
                                        ctypes.POINTER(bsa_route_spec), vp, ctypes.c_size_t, vp]
        L.bsa_decode_routed.restype = ctypes.c_int
        L.bsa_decode_routed_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, ctypes.c_int,
                                                f32, ctypes.POINTER(bsa_route_spec), vp]
        L.bsa_decode_routed_noalloc.restype = ctypes.c_int
        L.bsa_decode_workspace_bytes.argtypes = [i32, i32, i32]
        L.bsa_decode_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_build_route_transpose.argtypes = [vp, vp, i64, i64, vp, vp, vp]
        L.bsa_build_route_transpose.restype = ctypes.c_int
        L.bsa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, ctypes.c_int,
                                   f32, vp, vp, i64, vp, vp, vp, ctypes.c_size_t, vp]
        L.bsa_backward.restype = ctypes.c_int
        L.bsa_backward_workspace_bytes.argtypes = [i32, i32, i32, i64, i32, i32, i64]
        L.bsa_backward_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_bsbr_forward.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, ctypes.c_int, f32,
                                       vp, ctypes.c_size_t, vp]
        L.bsa_bsbr_forward.restype = ctypes.c_int
        L.bsa_bsbr_workspace_bytes.argtypes = [i32, i32, i32, i64, i32, i32]
        L.bsa_bsbr_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_check_route.argtypes = [vp, vp, i64, i64]
        L.bsa_check_route.restype = ctypes.c_int
        L.bsa_status_string.argtypes = [ctypes.c_int]
        L.bsa_status_string.restype = ctypes.c_char_p
        L.bsa_last_error.argtypes = []
        L.bsa_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().bsa_status_string(status).decode()


def bsa_status_string(status: int) -> str:
    return status_string(status)


def bsa_last_error() -> str:
    return lib().bsa_last_error().decode()


def _check(status: int) -> None:
    if status != BSA_OK:
        raise BsaError(status, bsa_last_error())


def _dev_ptr(t, name, dtype=None, allow_none=False):
    """Device pointer of a contiguous GPU tensor (or an int address, or None)."""
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype} (got {t.dtype})")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def route_spec(kind: int, n_local: int = 2, keep_first: int = 1, n_random: int = 14, seed: int = 17):
    return bsa_route_spec(kind, n_local, keep_first, n_random, seed)


def bsa_build_route(spec: bsa_route_spec, n: int, block: int, row_ptr=None, col_idx=None, stream=None) -> int:
    """Write the CSR route into row_ptr/col_idx (int32 GPU tensors); returns nnz.

    With row_ptr None this is the size query (no device work).
    """
    import torch
    nnz = ctypes.c_int64(0)
    if isinstance(col_idx, int):
        raise ValueError("pass col_idx as a tensor so its capacity is known")
    rp = _dev_ptr(row_ptr, "row_ptr", torch.int32, allow_none=True)
    ci = _dev_ptr(col_idx, "col_idx", torch.int32, allow_none=True) if rp is not None else None
    cap = col_idx.numel() if (rp is not None and col_idx is not None) else 0
    st = _stream(stream) if rp is not None else None
    _check(lib().bsa_build_route(ctypes.byref(spec), n, block, rp, ci, cap, ctypes.byref(nnz), st))
    return nnz.value


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BSA_BF16
    if t.dtype == torch.float32:
        return BSA_FP32
    raise ValueError(f"unsupported dtype {t.dtype}")


def bsa_forward(q, k, v, o, row_ptr, col_idx, block: int, scale: float = 0.0, lse=None, stream=None) -> None:
    """o = block-sparse attention(q, k, v) over the CSR route; q,o [b,Hq,n,d], k,v [b,Hkv,n,d]."""
    import torch
    dt = _dtype_code(q)
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    if tuple(k.shape) != (b, hkv, n, d) or tuple(v.shape) != (b, hkv, n, d) or tuple(o.shape) != (b, hq, n, d):
        raise ValueError("shape mismatch between q, k, v and o")
    ptrs = [_dev_ptr(x, nm, q.dtype) for x, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    if lse is not None and tuple(lse.shape) != (b, hq, n):
        raise ValueError("lse must have shape [b, Hq, n]")
    lp = _dev_ptr(lse, "lse", torch.float32, allow_none=True)
    rp = _dev_ptr(row_ptr, "row_ptr", torch.int32)
    ci = _dev_ptr(col_idx, "col_idx", torch.int32)
    nnz = col_idx.numel()
    _check(lib().bsa_forward(*ptrs, lp, b, hq, hkv, n, d, block, dt, float(scale), rp, ci, nnz, _stream(stream)))


def bsa_dense_route_workspace_bytes(n: int, block: int) -> int:
    return int(lib().bsa_dense_route_workspace_bytes(n, block))


def bsa_dense_causal_ref(q, k, v, o, workspace, block: int, scale: float = 0.0, lse=None, stream=None) -> None:
    """The same forward kernel over the dense causal route built into `workspace` (int32 GPU tensor)."""
    import torch
    dt = _dtype_code(q)
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    if tuple(k.shape) != (b, hkv, n, d) or tuple(v.shape) != (b, hkv, n, d) or tuple(o.shape) != (b, hq, n, d):
        raise ValueError("shape mismatch between q, k, v and o")
    ptrs = [_dev_ptr(x, nm, q.dtype) for x, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    lp = _dev_ptr(lse, "lse", torch.float32, allow_none=True)
    wp = _dev_ptr(workspace, "workspace", torch.int32)
    _check(lib().bsa_dense_causal_ref(*ptrs, lp, b, hq, hkv, n, d, block, dt, float(scale), wp,
                                      workspace.numel() * 4, _stream(stream)))


def bsa_decode_workspace_bytes(batch: int, heads_q: int, d: int) -> int:
    return int(lib().bsa_decode_workspace_bytes(batch, heads_q, d))


def bsa_decode(q, k_cache, v_cache, o, seq_lens, row_ptr, col_idx, block: int, workspace, scale: float = 0.0,
               lse=None, stream=None) -> None:
    """o[b, h] = attention of the newest token t = seq_lens[b] - 1 over its route row; q,o [b,Hq,d],
    k_cache,v_cache [b,Hkv,n_max,d], seq_lens int32 [b] (GPU), workspace float32 (GPU)."""
    import torch
    dt = _dtype_code(q)
    b, hq, d = q.shape
    hkv, n_max = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (b, hkv, n_max, d) or tuple(v_cache.shape) != (b, hkv, n_max, d) or \
            tuple(o.shape) != (b, hq, d):
        raise ValueError("shape mismatch between q, k_cache, v_cache and o")
    if tuple(seq_lens.shape) != (b,):
        raise ValueError("seq_lens must have shape [b]")
    if row_ptr.numel() != -(-n_max // block) + 1:
        raise ValueError("row_ptr must hold the route for n_max tokens (ceil(n_max / block) + 1 entries)")
    ptrs = [_dev_ptr(x, nm, q.dtype) for x, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (o, "o"))]
    if lse is not None and tuple(lse.shape) != (b, hq):
        raise ValueError("lse must have shape [b, Hq]")
    lp = _dev_ptr(lse, "lse", torch.float32, allow_none=True)
    sp = _dev_ptr(seq_lens, "seq_lens", torch.int32)
    rp = _dev_ptr(row_ptr, "row_ptr", torch.int32)
    ci = _dev_ptr(col_idx, "col_idx", torch.int32)
    wp = _dev_ptr(workspace, "workspace", torch.float32)
    _check(lib().bsa_decode(*ptrs, lp, sp, b, hq, hkv, n_max, d, block, dt, float(scale), rp, ci, col_idx.numel(),
                            wp, workspace.numel() * 4, _stream(stream)))


def bsa_decode_routed(q, k_cache, v_cache, o, seq_lens, spec: bsa_route_spec, block: int, workspace,
                      scale: float = 0.0, lse=None, stream=None) -> None:
    """bsa_decode with the route rows generated in the kernel from `spec` (no CSR route)."""
    import torch
    dt = _dtype_code(q)
    b, hq, d = q.shape
    hkv, n_max = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (b, hkv, n_max, d) or tuple(v_cache.shape) != (b, hkv, n_max, d) or \
            tuple(o.shape) != (b, hq, d):
        raise ValueError("shape mismatch between q, k_cache, v_cache and o")
    if tuple(seq_lens.shape) != (b,):
        raise ValueError("seq_lens must have shape [b]")
    ptrs = [_dev_ptr(x, nm, q.dtype) for x, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (o, "o"))]
    if lse is not None and tuple(lse.shape) != (b, hq):
        raise ValueError("lse must have shape [b, Hq]")
    lp = _dev_ptr(lse, "lse", torch.float32, allow_none=True)
    sp = _dev_ptr(seq_lens, "seq_lens", torch.int32)
    wp = _dev_ptr(workspace, "workspace", torch.float32)
    _check(lib().bsa_decode_routed(*ptrs, lp, sp, b, hq, hkv, n_max, d, block, dt, float(scale),
                                   ctypes.byref(spec), wp, workspace.numel() * 4, _stream(stream)))


def bsa_decode_routed_noalloc(q, k_cache, v_cache, o, seq_lens, spec: bsa_route_spec, block: int, scale: float = 0.0,
                              lse=None, stream=None) -> None:
    """bsa_decode_routed with its partials in the library's static scratch array (no workspace)."""
    import torch
    dt = _dtype_code(q)
    b, hq, d = q.shape
    hkv, n_max = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (b, hkv, n_max, d) or tuple(v_cache.shape) != (b, hkv, n_max, d) or \
            tuple(o.shape) != (b, hq, d):
        raise ValueError("shape mismatch between q, k_cache, v_cache and o")
    if tuple(seq_lens.shape) != (b,):
        raise ValueError("seq_lens must have shape [b]")
    ptrs = [_dev_ptr(x, nm, q.dtype) for x, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (o, "o"))]
    if lse is not None and tuple(lse.shape) != (b, hq):
        raise ValueError("lse must have shape [b, Hq]")
    lp = _dev_ptr(lse, "lse", torch.float32, allow_none=True)
    sp = _dev_ptr(seq_lens, "seq_lens", torch.int32)
    _check(lib().bsa_decode_routed_noalloc(*ptrs, lp, sp, b, hq, hkv, n_max, d, block, dt, float(scale),
                                           ctypes.byref(spec), _stream(stream)))


def bsa_build_route_transpose(row_ptr, col_idx, t_row_ptr, t_col_idx, stream=None) -> None:
    """Write the transposed route (readers of every key block) into t_row_ptr/t_col_idx (int32 GPU)."""
    import torch
    nqb = row_ptr.numel() - 1
    nnz = col_idx.numel()
    if t_row_ptr.numel() != nqb + 1 or t_col_idx.numel() != nnz:
        raise ValueError("t_row_ptr must have nqb + 1 entries and t_col_idx nnz entries")
    ptrs = [_dev_ptr(x, nm, torch.int32, allow_none=(x is None or x.numel() == 0))
            for x, nm in ((row_ptr, "row_ptr"), (col_idx, "col_idx"), (t_row_ptr, "t_row_ptr"), (t_col_idx, "t_col_idx"))]
    _check(lib().bsa_build_route_transpose(ptrs[0], ptrs[1], nqb, nnz, ptrs[2], ptrs[3], _stream(stream)))


def bsa_backward_workspace_bytes(batch: int, heads_q: int, heads_kv: int, n: int, d: int, block: int, nnz: int) -> int:
    return int(lib().bsa_backward_workspace_bytes(batch, heads_q, heads_kv, n, d, block, nnz))


def bsa_backward(q, k, v, o, d_o, lse, dq, dk, dv, row_ptr, col_idx, t_row_ptr, t_col_idx, block: int, workspace,
                 scale: float = 0.0, stream=None) -> None:
    """dq, dk, dv = gradients of bsa_forward for upstream gradient d_o (see include/bsa.h)."""
    import torch
    dt = _dtype_code(q)
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    for x, nm, shp in ((k, "k", (b, hkv, n, d)), (v, "v", (b, hkv, n, d)), (o, "o", (b, hq, n, d)),
                       (d_o, "d_o", (b, hq, n, d)), (dq, "dq", (b, hq, n, d)), (dk, "dk", (b, hkv, n, d)),
                       (dv, "dv", (b, hkv, n, d)), (lse, "lse", (b, hq, n))):
        if tuple(x.shape) != shp:
            raise ValueError(f"{nm} must have shape {shp}")
    ptrs = [_dev_ptr(x, nm, q.dtype) for x, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (d_o, "d_o"))]
    lp = _dev_ptr(lse, "lse", torch.float32)
    gp = [_dev_ptr(x, nm, q.dtype) for x, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    rp = _dev_ptr(row_ptr, "row_ptr", torch.int32)
    ci = _dev_ptr(col_idx, "col_idx", torch.int32)
    trp = _dev_ptr(t_row_ptr, "t_row_ptr", torch.int32)
    tci = _dev_ptr(t_col_idx, "t_col_idx", torch.int32)
    wp = _dev_ptr(workspace, "workspace")
    _check(lib().bsa_backward(*ptrs, lp, *gp, b, hq, hkv, n, d, block, dt, float(scale), rp, ci, col_idx.numel(),
                              trp, tci, wp, workspace.numel() * workspace.element_size(), _stream(stream)))


def build_route_transpose(row_ptr, col_idx, stream=None):
    """Allocate and build the transposed route on the GPU; returns (t_row_ptr, t_col_idx)."""
    import torch
    t_row_ptr = torch.empty_like(row_ptr)
    t_col_idx = torch.empty(max(col_idx.numel(), 1), dtype=torch.int32, device=col_idx.device)[:col_idx.numel()]
    bsa_build_route_transpose(row_ptr, col_idx, t_row_ptr, t_col_idx, stream)
    return t_row_ptr, t_col_idx


def backward(q, k, v, o, d_o, lse, row_ptr, col_idx, block: int, t_route=None, scale: float = 0.0, stream=None):
    """Allocate the gradients and workspace (and the transposed route unless given) and run bsa_backward."""
    import torch
    b, hq, n, d = q.shape
    t_row_ptr, t_col_idx = t_route if t_route is not None else build_route_transpose(row_ptr, col_idx, stream)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = bsa_backward_workspace_bytes(b, hq, k.shape[1], n, d, block, col_idx.numel())
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    bsa_backward(q, k, v, o, d_o, lse, dq, dk, dv, row_ptr, col_idx, t_row_ptr, t_col_idx, block, ws, scale, stream)
    return dq, dk, dv


def bsa_bsbr_workspace_bytes(batch: int, heads_q: int, heads_kv: int, n: int, d: int, chunk: int) -> int:
    return int(lib().bsa_bsbr_workspace_bytes(batch, heads_q, heads_kv, n, d, chunk))


def bsa_bsbr_forward(q, k, v, r_meta, h_meta, o, chunk: int, workspace, scale: float = 0.0, stream=None) -> None:
    """o = within-chunk attention + the BSBR retrieval over earlier chunks (see include/bsa.h)."""
    dt = _dtype_code(q)
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    nch = -(-n // chunk)
    for x, nm, shp in ((k, "k", (b, hkv, n, d)), (v, "v", (b, hkv, n, d)), (o, "o", (b, hq, n, d)),
                       (r_meta, "r_meta", (b, hq, nch, d)), (h_meta, "h_meta", (b, hkv, nch, d))):
        if tuple(x.shape) != shp:
            raise ValueError(f"{nm} must have shape {shp}")
    ptrs = [_dev_ptr(x, nm, q.dtype) for x, nm in ((q, "q"), (k, "k"), (v, "v"), (r_meta, "r_meta"),
                                                      (h_meta, "h_meta"), (o, "o"))]
    wp = _dev_ptr(workspace, "workspace")
    _check(lib().bsa_bsbr_forward(*ptrs, b, hq, hkv, n, d, chunk, dt, float(scale), wp,
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def bsbr_forward(q, k, v, r_meta, h_meta, chunk: int, scale: float = 0.0, stream=None):
    """Allocate the output and workspace and run bsa_bsbr_forward."""
    import torch
    b, hq, n, d = q.shape
    o = torch.empty_like(q)
    nbytes = bsa_bsbr_workspace_bytes(b, hq, k.shape[1], n, d, chunk)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    bsa_bsbr_forward(q, k, v, r_meta, h_meta, o, chunk, ws, scale, stream)
    return o


def bsa_check_route(row_ptr, col_idx) -> None:
    """Validate a CSR route held in host memory (numpy int32 arrays); raises BsaError if malformed."""
    import numpy as np
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    _check(lib().bsa_check_route(rp.ctypes.data, ci.ctypes.data if ci.size else None, len(rp) - 1, ci.size))


# --- small conveniences over the calls above (allocation via torch) ---------------------------

def build_route(spec: bsa_route_spec, n: int, block: int, device="cuda", stream=None):
    """Allocate and build a route on the GPU; returns (row_ptr, col_idx) int32 tensors."""
    import torch
    nnz = bsa_build_route(spec, n, block)
    nqb = -(-n // block)
    row_ptr = torch.empty(nqb + 1, dtype=torch.int32, device=device)
    col_idx = torch.empty(max(nnz, 1), dtype=torch.int32, device=device)[:nnz]
    bsa_build_route(spec, n, block, row_ptr, col_idx, stream)
    return row_ptr, col_idx


def decode(q, k_cache, v_cache, seq_lens, row_ptr, col_idx, block: int, scale: float = 0.0,
           with_lse: bool = False, stream=None):
    """Allocate the output, LSE and workspace and run bsa_decode."""
    import torch
    b, hq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(b, hq, dtype=torch.float32, device=q.device) if with_lse else None
    ws = torch.empty(max(1, bsa_decode_workspace_bytes(b, hq, d) // 4), dtype=torch.float32, device=q.device)
    bsa_decode(q, k_cache, v_cache, o, seq_lens, row_ptr, col_idx, block, ws, scale, lse, stream)
    return (o, lse) if with_lse else o


def decode_routed(q, k_cache, v_cache, seq_lens, spec: bsa_route_spec, block: int, scale: float = 0.0,
                  with_lse: bool = False, stream=None):
    """Allocate the output, LSE and workspace and run bsa_decode_routed."""
    import torch
    b, hq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(b, hq, dtype=torch.float32, device=q.device) if with_lse else None
    ws = torch.empty(max(1, bsa_decode_workspace_bytes(b, hq, d) // 4), dtype=torch.float32, device=q.device)
    bsa_decode_routed(q, k_cache, v_cache, o, seq_lens, spec, block, ws, scale, lse, stream)
    return (o, lse) if with_lse else o


def forward(q, k, v, row_ptr, col_idx, block: int, scale: float = 0.0, with_lse: bool = False, stream=None):
    """Allocate the output (and LSE) and run bsa_forward."""
    import torch
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if with_lse else None
    bsa_forward(q, k, v, o, row_ptr, col_idx, block, scale, lse, stream)
    return (o, lse) if with_lse else o
