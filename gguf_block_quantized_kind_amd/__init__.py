"""Python binding of libqmm: matmul against GGUF block-quantized weights on
AMD MI355X (gfx950).

The functions named ``qmm_*`` mirror the C entry points of include/qmm.h one
for one.  They only marshal arguments: torch tensors (device memory) become
pointers, a torch stream (default: the current one) becomes the hipStream_t,
and a non-zero status becomes a QmmError.  Every step of the computation runs
in the HIP kernels of libqmm.so; if that library has not been built, loading
it raises instead of falling back to anything else.

``gemv``, ``gemm``, ``matmul``, ``moe`` and ``dequant`` are conveniences that
allocate their outputs (and the expert workspace) with torch and call the
``qmm_*`` functions.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libqmm.so")

QMM_F32, QMM_F16 = 0, 1
GEMV_MAX_M = 8
KIND_NAMES = ("Q8_0", "Q4_0", "Q5_0", "Q2_K", "Q3_K", "Q4_K", "Q5_K", "Q6_K",
              "IQ4_NL", "IQ4_XS", "MXFP4")


class QmmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"qmm status {status}: {message}")
        self.status = status
        self.message = message


_lib = None


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Loads libqmm.so (no fallback: a missing library is an error)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950) first")
    lib = ctypes.CDLL(path)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "qmm_gemv": (I, [I, P, P, P, I64, I64]),
        "qmm_gemv_ex": (I, [I, P, P, I, P, I64, I64, I64, P]),
        "qmm_gemm": (I, [I, P, P, P, I64, I64, I64]),
        "qmm_gemm_ex": (I, [I, P, P, I, P, I64, I64, I64, P]),
        "qmm_matmul": (I, [I, P, P, I, P, I64, I64, I64, P]),
        "qmm_moe": (I, [I, P, I64, P, I64, P, I, I, P, I64, I64, I64, P, SZ, P]),
        "qmm_moe_workspace_bytes": (SZ, [I64, I64, I64]),
        "qmm_gemm_mx": (I, [I, P, P, I, P, I64, I64, I64, P, SZ, P]),
        "qmm_moe_ffn": (I, [I, P, P, I64, P, P, I64, P, I, P, I64, I64, I64, P, SZ, P]),
        "qmm_moe_ffn_packed": (I, [I, P, P, I64, P, P, I64, P, I, P, I64, I64, I64, P, SZ, P]),
        "qmm_moe_ffn_workspace_bytes": (SZ, [I64, I64, I64, I64, I64]),
        "qmm_gemm_mx_workspace_bytes": (SZ, [I64, I64]),
        "qmm_dequant": (I, [I, P, P, I64, P]),
        "qmm_packed_bytes": (I64, [I, I64, I64]),
        "qmm_repack": (I, [I, P, P, I64, I64, P]),
        "qmm_gemv_packed": (I, [I, P, P, I, P, I64, I64, I64, P]),
        "qmm_gemv_i8": (I, [I, P, P, I, P, I64, I64, I64, P, SZ, P]),
        "qmm_matmul_packed": (I, [I, P, P, I, P, I64, I64, I64, P]),
        "qmm_gemv_i8_noalloc": (I, [I, P, P, I, P, I64, I64, I64, P]),
        "qmm_moe_packed": (I, [I, P, I64, P, I64, P, I, I, P, I64, I64, I64, P, SZ, P]),
        "qmm_gemv_i8_workspace_bytes": (SZ, [I64, I64]),
        "qmm_row_bytes": (I64, [I, I64]),
        "qmm_block_geometry": (I, [I, ctypes.POINTER(I), ctypes.POINTER(I)]),
        "qmm_kind_from_name": (I, [ctypes.c_char_p]),
        "qmm_kind_name": (ctypes.c_char_p, [I]),
        "qmm_status_string": (ctypes.c_char_p, [I]),
        "qmm_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise QmmError(status, (lib.qmm_last_error() or b"").decode() or
                       lib.qmm_status_string(status).decode())


# ---------------------------------------------------------------------------
# Names and geometry
# ---------------------------------------------------------------------------
def qmm_kind_from_name(name: str) -> int:
    return int(load_library().qmm_kind_from_name(name.encode()))


def qmm_kind_name(kind: int):
    r = load_library().qmm_kind_name(int(kind))
    return None if r is None else r.decode()


def qmm_row_bytes(kind, K: int) -> int:
    return int(load_library().qmm_row_bytes(kind_id(kind), int(K)))


def qmm_block_geometry(kind) -> tuple[int, int]:
    b, e = ctypes.c_int(), ctypes.c_int()
    _check(load_library().qmm_block_geometry(kind_id(kind), ctypes.byref(b), ctypes.byref(e)))
    return b.value, e.value


def qmm_status_string(status: int) -> str:
    return load_library().qmm_status_string(int(status)).decode()


def qmm_last_error() -> str:
    return (load_library().qmm_last_error() or b"").decode()


def qmm_moe_workspace_bytes(E: int, M: int, topk: int) -> int:
    return int(load_library().qmm_moe_workspace_bytes(int(E), int(M), int(topk)))


def qmm_moe_ffn_workspace_bytes(E: int, M: int, topk: int, N_ff: int, K: int) -> int:
    return int(load_library().qmm_moe_ffn_workspace_bytes(int(E), int(M), int(topk), int(N_ff), int(K)))


def qmm_gemm_mx_workspace_bytes(M: int, K: int) -> int:
    return int(load_library().qmm_gemm_mx_workspace_bytes(int(M), int(K)))


def kind_id(kind) -> int:
    if isinstance(kind, str):
        k = qmm_kind_from_name(kind)
        if k < 0:
            raise QmmError(2, f"{kind} is not one of the eleven supported kinds")
        return k
    return int(kind)


# ---------------------------------------------------------------------------
# Tensor marshalling
# ---------------------------------------------------------------------------
def _ptr(t) -> int:
    """Device address of a tensor; a host tensor is refused (the kernels
    would fault on its address)."""
    if t is None:
        return 0
    if t.device.type != "cuda":
        raise ValueError(f"a {tuple(t.shape)} tensor is on {t.device}: the library takes device memory only")
    return int(t.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return QMM_F32
    if t.dtype == torch.float16:
        return QMM_F16
    return 99  # refused by the library as a bad dtype


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


_F32, _F16, _F32_OR_F16, _I32 = ("float32",), ("float16",), ("float32", "float16"), ("int32",)


def _need(t, count: int, what: str, dtypes=None):
    """Length, layout and element type of a buffer the library will touch:
    a wrong element type would make the counts below mean other byte sizes
    (an f16 output of M*N elements is half the bytes the kernel writes)."""
    if t is None:
        return
    if dtypes is not None and str(t.dtype).replace("torch.", "") not in dtypes:
        raise TypeError(f"{what} must be {' or '.join(dtypes)}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() < count:
        raise ValueError(f"{what} holds {t.numel()} elements, needs {count}")


def _check_weights(kind, W, rows: int, K: int):
    if W is not None and W.element_size() != 1:
        raise TypeError(f"W must be a byte tensor (uint8 or int8), got {W.dtype}")
    rb = qmm_row_bytes(kind, K)
    if rb > 0:
        _need(W, rows * rb, "W (bytes)")


# ---------------------------------------------------------------------------
# The C entry points
# ---------------------------------------------------------------------------
def qmm_gemv(kind, W, x, y, N: int, K: int):
    _check_weights(kind, W, N, K)
    _need(x, K, "x", _F32)
    _need(y, N, "y", _F32)
    _check(load_library().qmm_gemv(kind_id(kind), _ptr(W), _ptr(x), _ptr(y), N, K))


def qmm_gemv_ex(kind, W, x, y, M: int, N: int, K: int, stream=None):
    _check_weights(kind, W, N, K)
    _need(x, M * K, "x", _F32_OR_F16)
    _need(y, M * N, "y", _F32)
    _check(load_library().qmm_gemv_ex(kind_id(kind), _ptr(W), _ptr(x), _dtype_code(x), _ptr(y),
                                      M, N, K, _stream(stream)))


def qmm_gemm(kind, W, A, C, M: int, N: int, K: int):
    _check_weights(kind, W, N, K)
    _need(A, M * K, "A", _F16)
    _need(C, M * N, "C", _F32)
    _check(load_library().qmm_gemm(kind_id(kind), _ptr(W), _ptr(A), _ptr(C), M, N, K))


def qmm_gemm_ex(kind, W, A, C, M: int, N: int, K: int, stream=None):
    _check_weights(kind, W, N, K)
    _need(A, M * K, "A", _F32_OR_F16)
    _need(C, M * N, "C", _F32)
    _check(load_library().qmm_gemm_ex(kind_id(kind), _ptr(W), _ptr(A), _dtype_code(A), _ptr(C),
                                      M, N, K, _stream(stream)))


def qmm_matmul(kind, W, A, C, M: int, N: int, K: int, stream=None):
    _check_weights(kind, W, N, K)
    _need(A, M * K, "A", _F32_OR_F16)
    _need(C, M * N, "C", _F32)
    _check(load_library().qmm_matmul(kind_id(kind), _ptr(W), _ptr(A), _dtype_code(A), _ptr(C),
                                     M, N, K, _stream(stream)))


def qmm_gemm_mx(kind, W, A, C, M: int, N: int, K: int, workspace, stream=None):
    _check_weights(kind, W, N, K)
    _need(A, M * K, "A", _F32_OR_F16)
    _need(C, M * N, "C", _F32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().qmm_gemm_mx(kind_id(kind), _ptr(W), _ptr(A), _dtype_code(A), _ptr(C),
                                      M, N, K, _ptr(workspace), ws_bytes, _stream(stream)))


def qmm_moe_ffn(kind, W_gu, W_d, E: int, ids, topk_w, topk: int, X, Y, M: int, N_ff: int, K: int,
                workspace, stream=None):
    _check_weights(kind, W_gu, E * 2 * N_ff, K)
    _check_weights(kind, W_d, E * K, N_ff)
    _need(ids, M * topk, "ids", _I32)
    _need(topk_w, M * topk, "topk_w", _F32)
    _need(X, M * K, "X", _F32_OR_F16)
    _need(Y, M * K, "Y", _F32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().qmm_moe_ffn(kind_id(kind), _ptr(W_gu), _ptr(W_d), E, _ptr(ids), _ptr(topk_w), topk,
                                      _ptr(X), _dtype_code(X), _ptr(Y), M, N_ff, K, _ptr(workspace), ws_bytes,
                                      _stream(stream)))


def _check_packed_bytes(kind, P, count: int, N: int, K: int, what: str):
    pb = qmm_packed_bytes(kind, N, K)
    if P is not None and P.element_size() != 1:
        raise TypeError(f"{what} must be a byte tensor, got {P.dtype}")
    if pb > 0:
        _need(P, count * pb, f"{what} (bytes)")


def qmm_moe_ffn_packed(kind, P_gu, P_d, E: int, ids, topk_w, topk: int, X, Y, M: int, N_ff: int, K: int,
                       workspace, stream=None):
    _check_packed_bytes(kind, P_gu, E, 2 * N_ff, K, "P_gu")
    _check_packed_bytes(kind, P_d, E, K, N_ff, "P_d")
    _need(ids, M * topk, "ids", _I32)
    _need(topk_w, M * topk, "topk_w", _F32)
    _need(X, M * K, "X", _F32_OR_F16)
    _need(Y, M * K, "Y", _F32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().qmm_moe_ffn_packed(kind_id(kind), _ptr(P_gu), _ptr(P_d), E, _ptr(ids), _ptr(topk_w),
                                             topk, _ptr(X), _dtype_code(X), _ptr(Y), M, N_ff, K, _ptr(workspace),
                                             ws_bytes, _stream(stream)))


def qmm_moe(kind, W, E: int, ids, topk: int, X, x_per_slot: int, Y, M: int, N: int, K: int,
            workspace, stream=None):
    _check_weights(kind, W, E * N, K)
    _need(ids, M * topk, "ids", _I32)
    _need(X, M * (topk if x_per_slot else 1) * K, "X", _F32_OR_F16)
    _need(Y, M * topk * N, "Y", _F32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().qmm_moe(kind_id(kind), _ptr(W), E, _ptr(ids), topk, _ptr(X),
                                  _dtype_code(X), int(x_per_slot), _ptr(Y), M, N, K,
                                  _ptr(workspace), ws_bytes, _stream(stream)))


def qmm_packed_bytes(kind, N: int, K: int) -> int:
    return int(load_library().qmm_packed_bytes(kind_id(kind), N, K))


def qmm_repack(kind, W, P, N: int, K: int, stream=None):
    _check_weights(kind, W, N, K)
    pb = qmm_packed_bytes(kind, N, K)
    if P is not None and P.element_size() != 1:
        raise TypeError(f"P must be a byte tensor, got {P.dtype}")
    if pb > 0:
        _need(P, pb, "P (bytes)")
    _check(load_library().qmm_repack(kind_id(kind), _ptr(W), _ptr(P), N, K, _stream(stream)))


def qmm_gemv_packed(kind, P, x, y, M: int, N: int, K: int, stream=None):
    pb = qmm_packed_bytes(kind, N, K)
    if P is not None and P.element_size() != 1:
        raise TypeError(f"P must be a byte tensor, got {P.dtype}")
    if pb > 0:
        _need(P, pb, "P (bytes)")
    _need(x, M * K, "x", _F32_OR_F16)
    _need(y, M * N, "y", _F32)
    _check(load_library().qmm_gemv_packed(kind_id(kind), _ptr(P), _ptr(x), _dtype_code(x), _ptr(y),
                                          M, N, K, _stream(stream)))


def qmm_matmul_packed(kind, P, A, C, M: int, N: int, K: int, stream=None):
    pb = qmm_packed_bytes(kind, N, K)
    if P is not None and P.element_size() != 1:
        raise TypeError(f"P must be a byte tensor, got {P.dtype}")
    if pb > 0:
        _need(P, pb, "P (bytes)")
    _need(A, M * K, "A", _F32_OR_F16)
    _need(C, M * N, "C", _F32)
    _check(load_library().qmm_matmul_packed(kind_id(kind), _ptr(P), _ptr(A), _dtype_code(A), _ptr(C),
                                            M, N, K, _stream(stream)))


def qmm_moe_packed(kind, P, E: int, ids, topk: int, X, x_per_slot: int, Y, M: int, N: int, K: int,
                   workspace, stream=None):
    pb = qmm_packed_bytes(kind, N, K)
    if P is not None and P.element_size() != 1:
        raise TypeError(f"P must be a byte tensor, got {P.dtype}")
    if pb > 0:
        _need(P, E * pb, "P (bytes)")
    _need(ids, M * topk, "ids", _I32)
    _need(X, (M * topk if x_per_slot else M) * K, "X", _F32_OR_F16)
    _need(Y, M * topk * N, "Y", _F32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().qmm_moe_packed(kind_id(kind), _ptr(P), E, _ptr(ids), topk, _ptr(X), _dtype_code(X),
                                         int(bool(x_per_slot)), _ptr(Y), M, N, K, _ptr(workspace), ws_bytes,
                                         _stream(stream)))


def qmm_gemv_i8_workspace_bytes(M: int, K: int) -> int:
    return int(load_library().qmm_gemv_i8_workspace_bytes(M, K))


def qmm_gemv_i8(kind, P, x, y, M: int, N: int, K: int, workspace, stream=None):
    pb = qmm_packed_bytes(kind, N, K)
    if P is not None and P.element_size() != 1:
        raise TypeError(f"P must be a byte tensor, got {P.dtype}")
    if pb > 0:
        _need(P, pb, "P (bytes)")
    _need(x, M * K, "x", _F32_OR_F16)
    _need(y, M * N, "y", _F32)
    if workspace is not None and workspace.element_size() != 1:
        raise TypeError(f"workspace must be a byte tensor, got {workspace.dtype}")
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(load_library().qmm_gemv_i8(kind_id(kind), _ptr(P), _ptr(x), _dtype_code(x), _ptr(y), M, N, K,
                                      _ptr(workspace), ws_bytes, _stream(stream)))


def qmm_gemv_i8_noalloc(kind, P, x, y, M: int, N: int, K: int, stream=None):
    """qmm_gemv_i8 on the library's own device scratch (no workspace; calls
    that overlap on one GPU race on it)."""
    pb = qmm_packed_bytes(kind, N, K)
    if P is not None and P.element_size() != 1:
        raise TypeError(f"P must be a byte tensor, got {P.dtype}")
    if pb > 0:
        _need(P, pb, "P (bytes)")
    _need(x, M * K, "x", _F32_OR_F16)
    _need(y, M * N, "y", _F32)
    _check(load_library().qmm_gemv_i8_noalloc(kind_id(kind), _ptr(P), _ptr(x), _dtype_code(x), _ptr(y), M, N, K,
                                              _stream(stream)))


def qmm_dequant(kind, W, out, n_elems: int, stream=None):
    bb, be = qmm_block_geometry(kind)
    if n_elems % be == 0:
        if W is not None and W.element_size() != 1:
            raise TypeError(f"W must be a byte tensor (uint8 or int8), got {W.dtype}")
        _need(W, (n_elems // be) * bb, "W (bytes)")
    _need(out, n_elems, "out", _F32)
    _check(load_library().qmm_dequant(kind_id(kind), _ptr(W), _ptr(out), n_elems, _stream(stream)))


# ---------------------------------------------------------------------------
# Conveniences that allocate their outputs with torch
# ---------------------------------------------------------------------------
def _rows_of(kind, W, K: int) -> int:
    return (W.numel() // qmm_row_bytes(kind, K))


def gemv(kind, W, x, N: int | None = None, stream=None):
    """y[M, N] for x [M, K] (M <= 8) or [K]."""
    import torch
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    M, K = x2.shape
    N = _rows_of(kind, W, K) if N is None else N
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    qmm_gemv_ex(kind, W, x2, y, M, N, K, stream)
    return y


def gemm(kind, W, A, N: int | None = None, stream=None):
    import torch
    M, K = A.shape
    N = _rows_of(kind, W, K) if N is None else N
    C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    qmm_gemm_ex(kind, W, A, C, M, N, K, stream)
    return C


def matmul(kind, W, A, N: int | None = None, stream=None):
    import torch
    M, K = A.shape
    N = _rows_of(kind, W, K) if N is None else N
    C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    qmm_matmul(kind, W, A, C, M, N, K, stream)
    return C


def gemm_mx(kind, W, A, N: int | None = None, stream=None, workspace=None):
    """C [M, N] from MXFP4 weights with A quantized to MX FP8 (scaled FP4 matrix cores)."""
    import torch
    M, K = A.shape
    N = _rows_of(kind, W, K) if N is None else N
    C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if workspace is None:
        nbytes = qmm_gemm_mx_workspace_bytes(M, K)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=A.device)
    qmm_gemm_mx(kind, W, A, C, M, N, K, workspace, stream)
    return C


def moe(kind, W, E: int, ids, X, N: int, K: int, x_per_slot: bool, stream=None, workspace=None):
    """Y [M, topk, N] for ids [M, topk] int32 and X [M, K] or [M, topk, K]."""
    import torch
    M, topk = ids.shape
    Y = torch.empty((M, topk, N), dtype=torch.float32, device=X.device)
    if workspace is None:
        nbytes = qmm_moe_workspace_bytes(E, M, topk)
        workspace = torch.empty((nbytes + 3) // 4, dtype=torch.int32, device=X.device)
    qmm_moe(kind, W, E, ids, topk, X, 1 if x_per_slot else 0, Y, M, N, K, workspace, stream)
    return Y


def moe_ffn(kind, W_gu, W_d, E: int, ids, topk_w, X, N_ff: int, stream=None, workspace=None):
    """Y [M, K] = sum over slots of topk_w * down(silu(gate) * up) for ids [M, topk] int32,
    topk_w [M, topk] f32 and X [M, K]."""
    import torch
    M, topk = ids.shape
    K = X.shape[1]
    Y = torch.empty((M, K), dtype=torch.float32, device=X.device)
    if workspace is None:
        nbytes = qmm_moe_ffn_workspace_bytes(E, M, topk, N_ff, K)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=X.device)
    qmm_moe_ffn(kind, W_gu, W_d, E, ids, topk_w, topk, X, Y, M, N_ff, K, workspace, stream)
    return Y


def moe_ffn_packed(kind, P_gu, P_d, E: int, ids, topk_w, X, N_ff: int, stream=None, workspace=None):
    """moe_ffn over experts repacked with repack_experts (gate/up: E experts of
    2 N_ff rows of K; down: E experts of K rows of N_ff)."""
    import torch
    M, topk = ids.shape
    K = X.shape[1]
    Y = torch.empty((M, K), dtype=torch.float32, device=X.device)
    if workspace is None:
        nbytes = qmm_moe_ffn_workspace_bytes(E, M, topk, N_ff, K)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=X.device)
    qmm_moe_ffn_packed(kind, P_gu, P_d, E, ids, topk_w, topk, X, Y, M, N_ff, K, workspace, stream)
    return Y


def repack(kind, W, N: int, K: int, stream=None):
    """The repacked layout of N native rows (a new uint8 tensor)."""
    import torch
    pb = qmm_packed_bytes(kind, N, K)
    if pb < 0:  # the library names the reason (kind, K or shape)
        _check(load_library().qmm_repack(kind_id(kind), None, None, N, K, None))
        raise QmmError(5, f"kind {kind} with N={N}, K={K} has no repacked layout")
    P = torch.empty(pb, dtype=torch.uint8, device=W.device)
    qmm_repack(kind, W, P, N, K, stream)
    return P


def gemv_packed(kind, P, x, N: int, stream=None):
    """y[M, N] for x [M, K] (M <= 8) or [K], from repacked weights."""
    import torch
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    M, K = x2.shape
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    qmm_gemv_packed(kind, P, x2, y, M, N, K, stream)
    return y


def repack_experts(kind, W, E: int, N: int, K: int, stream=None):
    """E experts of N native rows each, repacked one by one (expert e's
    records at e * qmm_packed_bytes(kind, N, K))."""
    import torch
    pb = qmm_packed_bytes(kind, N, K)
    if pb < 0:
        _check(load_library().qmm_repack(kind_id(kind), None, None, N, K, None))
        raise QmmError(5, f"kind {kind} with N={N}, K={K} has no repacked layout")
    rb = qmm_row_bytes(kind, K)
    _check_weights(kind, W, E * N, K)
    P = torch.empty(E * pb, dtype=torch.uint8, device=W.device)
    Wf = W.reshape(-1)
    for e in range(E):
        qmm_repack(kind, Wf[e * N * rb:(e + 1) * N * rb], P[e * pb:(e + 1) * pb], N, K, stream)
    return P


def moe_packed(kind, P, E: int, ids, X, N: int, K: int, x_per_slot: bool, stream=None, workspace=None):
    """Y[M, topk, N] of the routed expert products over repacked experts."""
    import torch
    M, topk = ids.shape
    Y = torch.empty((M, topk, N), dtype=torch.float32, device=X.device)
    if workspace is None:
        nbytes = qmm_moe_workspace_bytes(E, M, topk)
        workspace = torch.empty((nbytes + 3) // 4, dtype=torch.int32, device=X.device)
    qmm_moe_packed(kind, P, E, ids, topk, X, int(x_per_slot), Y, M, N, K, workspace, stream)
    return Y


def gemv_i8(kind, P, x, N: int, stream=None, workspace=None):
    """y[M, N] from repacked Q8_0 / Q4_0 weights with int8-quantized x."""
    import torch
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    M, K = x2.shape
    if workspace is None:
        workspace = torch.empty(max(qmm_gemv_i8_workspace_bytes(M, K), 1), dtype=torch.uint8, device=x.device)
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    qmm_gemv_i8(kind, P, x2, y, M, N, K, workspace, stream)
    return y


def dequant(kind, W, n_elems: int | None = None, stream=None):
    import torch
    bb, be = qmm_block_geometry(kind)
    n = (W.numel() // bb) * be if n_elems is None else n_elems
    out = torch.empty(n, dtype=torch.float32, device=W.device)
    qmm_dequant(kind, W, out, n, stream)
    return out
