"""Thin Python binding of libnmsparse (ctypes).

Argument marshalling only: every function checks device, dtype and layout of
its torch tensors, allocates outputs with torch when none are given, and calls
the C ABI on torch's current HIP stream.  Every step of the computation runs
in the library's gfx950 kernels; nothing here computes, and there is no CPU
fallback -- a missing library or a CPU tensor is an error.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnmsparse.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "nmsparse.h")

NM_OK, NM_ERR_NULL, NM_ERR_SHAPE, NM_ERR_UNSUPPORTED, NM_ERR_ALIGN, NM_ERR_HIP, NM_ERR_TOO_LARGE = range(7)
NM_F32, NM_BF16 = 0, 1

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p

# name -> argument types, in header order
_SIGNATURES = {
    "nm_prune": [_int, _vp, _i64, _i64, _i64, _int, _int, _vp, _i64, _vp],
    "nm_compress": [_int, _vp, _i64, _vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp],
    "nm_prune_compress": [_int, _vp, _i64, _i64, _i64, _int, _int, _vp, _i64, _vp, _vp, _vp],
    "nm_reprune_t_transpose": [_int, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp],
    "nm_prune_compress_transpose": [_int, _vp, _i64, _i64, _i64, _int, _int, _vp, _i64, _vp, _vp, _vp, _i64, _i64,
                                    _i64, _vp, _i64, _vp],
    "nm_decompress": [_int, _vp, _vp, _i64, _i64, _int, _int, _vp, _i64, _vp],
    "spmm_nm": [_int, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp],
    "spmm_nm_t": [_int, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp],
    "nm_to_panels": [_int, _vp, _vp, _i64, _i64, _vp, _vp, _vp],
    "nm_mfma_rate_probe": [_int, _i64, _vp, ctypes.POINTER(_i64), _vp],
    "nm_reprune_t_transpose_panels": [_int, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp],
    "spmm_nm_t_panels": [_int, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp],
    "spmm_nm_t_out_bf16": [_int, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp],
    "spmm_nm_t_lowrank": [_int, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _i64,
                          _vp],
    "spmm_nm_t_relu_venom": [_int, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp],
    "spmm_nm_general": [_int, _vp, _vp, _i64, _i64, _int, _int, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp],
    "spmm_nm_general_noalloc": [_int, _vp, _vp, _i64, _i64, _int, _int, _vp, _i64, _i64, _vp, _i64, _vp],
    "sddmm_venom": [_int, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _int, _vp, _vp, _i64,
                    _vp],
    "spmm_venom_tn": [_int, _vp, _vp, _vp, _i64, _i64, _int, _int, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp],
    "nm_transpose": [_int, _vp, _i64, _i64, _i64, _vp, _i64, _vp],
    "prune_act_venom": [_int, _vp, _i64, _i64, _i64, _int, _int, _int, _vp, _vp, _vp, _vp, _i64, _vp],
    "spmm_venom": [_int, _vp, _vp, _vp, _i64, _i64, _int, _int, _vp, _i64, _i64, _vp, _i64, _vp],
    "nm_reprune_t": [_int, _vp, _vp, _i64, _i64, _vp, _vp, _vp],
    "sddmm_nm": [_int, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp],
    "sddmm_nm_dt": [_int, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp],
}

_lib = None


class NmError(RuntimeError):
    """A non-OK status returned by libnmsparse."""

    def __init__(self, status: int, call: str):
        self.status = status
        msg = lib().nm_status_str(status).decode()
        if status == NM_ERR_HIP:
            msg += ": " + lib().nm_last_hip_error().decode()
        super().__init__(f"{call}: {msg} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_matmul_ffns_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.nm_sizes.argtypes = [_i64, _i64, _int, _int, _int, ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                               ctypes.POINTER(_i64)]
        L.nm_sizes.restype = None
        L.nm_general_work_bytes.argtypes = [_int, _i64, _i64, _int, _int]
        L.nm_general_work_bytes.restype = _i64
        L.nm_venom_tn_work_bytes.argtypes = [_int, _i64, _i64]
        L.nm_venom_tn_work_bytes.restype = _i64
        L.nm_gmp_n_at.argtypes = [_int, _int, _i64, _i64, _i64, _i64, _i64, ctypes.POINTER(_int)]
        L.nm_gmp_n_at.restype = _int
        L.nm_general_scratch_bytes.argtypes = []
        L.nm_general_scratch_bytes.restype = _i64
        L.nm_status_str.argtypes = [_int]
        L.nm_status_str.restype = ctypes.c_char_p
        L.nm_last_hip_error.argtypes = []
        L.nm_last_hip_error.restype = ctypes.c_char_p
        L.nm_version.argtypes = []
        L.nm_version.restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/nmsparse.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:nm_status|void|const char\*|int|int64_t)\s+(\w+)\s*\(", text, flags=re.M)


def _check(status: int, call: str) -> None:
    if status != NM_OK:
        raise NmError(status, call)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return NM_BF16
    if t.dtype == torch.float32:
        return NM_F32
    raise TypeError(f"unsupported dtype {t.dtype}: bfloat16 or float32")


def _dev(*ts: torch.Tensor) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libnmsparse works on GPU tensors only (no CPU fallback)")


def _rows(t: torch.Tensor, name: str) -> int:
    """Row stride of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with contiguous rows")
    return t.stride(0)


def _flat(t: torch.Tensor, name: str) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _p(t):
    return None if t is None else t.data_ptr()


def sizes(R: int, K: int, N: int = 2, M: int = 4, V: int = 0):
    """(n_values, meta_bytes, colsel_bytes) of the compressed form (host-only)."""
    a, b, c = _i64(), _i64(), _i64()
    lib().nm_sizes(R, K, N, M, V, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return a.value, b.value, c.value


def nm_prune(A: torch.Tensor, N: int = 2, M: int = 4, mask: torch.Tensor | None = None) -> torch.Tensor:
    _dev(A, mask)
    R, K = A.shape
    lda = _rows(A, "A")
    if mask is None:
        mask = torch.empty((R, K), dtype=torch.uint8, device=A.device)
    _check(lib().nm_prune(_dt(A), _p(A), lda, R, K, N, M, _p(mask), _rows(mask, "mask"), _stream()), "nm_prune")
    return mask


def nm_compress(A: torch.Tensor, mask: torch.Tensor, N: int = 2, M: int = 4,
                bad_groups: torch.Tensor | None = None, values=None, meta=None):
    _dev(A, mask, bad_groups, values, meta)
    R, K = A.shape
    nv, mb, _ = sizes(R, K, N, M)
    if values is None:
        values = torch.empty((R, nv // R), dtype=A.dtype, device=A.device)
    if meta is None:
        meta = torch.empty((R, mb // R), dtype=torch.uint8, device=A.device)
    _flat(values, "values"), _flat(meta, "meta")
    _check(lib().nm_compress(_dt(A), _p(A), _rows(A, "A"), _p(mask), _rows(mask, "mask"), R, K, N, M,
                             _p(values), _p(meta), _p(bad_groups), _stream()), "nm_compress")
    return values, meta


def nm_prune_compress(A: torch.Tensor, N: int = 2, M: int = 4, mask=None, values=None, meta=None):
    """nm_prune and nm_compress in one call: returns (mask, values, meta)."""
    _dev(A, mask, values, meta)
    R, K = A.shape
    nv, mb, _ = sizes(R, K, N, M)
    if mask is None:
        mask = torch.empty((R, K), dtype=torch.uint8, device=A.device)
    if values is None:
        values = torch.empty((R, nv // R), dtype=A.dtype, device=A.device)
    if meta is None:
        meta = torch.empty((R, mb // R), dtype=torch.uint8, device=A.device)
    _flat(values, "values"), _flat(meta, "meta")
    _check(lib().nm_prune_compress(_dt(A), _p(A), _rows(A, "A"), R, K, N, M, _p(mask), _rows(mask, "mask"),
                                   _p(values), _p(meta), _stream()), "nm_prune_compress")
    return mask, values, meta


def nm_prune_compress_transpose(A: torch.Tensor, B: torch.Tensor, N: int = 2, M: int = 4, mask=None, values=None,
                                meta=None, Bt=None):
    """nm_prune_compress(A) and transpose(B) in one launch (bf16): returns (mask, values, meta, Bt)."""
    _dev(A, B, mask, values, meta, Bt)
    R, K = A.shape
    KB, Nc = B.shape
    nv, mb, _ = sizes(R, K, N, M)
    if mask is None:
        mask = torch.empty((R, K), dtype=torch.uint8, device=A.device)
    if values is None:
        values = torch.empty((R, nv // R), dtype=A.dtype, device=A.device)
    if meta is None:
        meta = torch.empty((R, mb // R), dtype=torch.uint8, device=A.device)
    if Bt is None:
        Bt = torch.empty((Nc, KB), dtype=B.dtype, device=B.device)
    if Bt.shape != (Nc, KB) or Bt.dtype != B.dtype:
        raise ValueError("Bt must be [Nc, KB] with B's dtype")
    if A.dtype != B.dtype:
        raise ValueError("A and B must share a dtype")
    _flat(values, "values"), _flat(meta, "meta")
    _check(lib().nm_prune_compress_transpose(_dt(A), _p(A), _rows(A, "A"), R, K, N, M, _p(mask), _rows(mask, "mask"),
                                             _p(values), _p(meta), _p(B), _rows(B, "B"), KB, Nc, _p(Bt),
                                             _rows(Bt, "Bt"), _stream()), "nm_prune_compress_transpose")
    return mask, values, meta, Bt


def nm_decompress(values: torch.Tensor, meta: torch.Tensor, K: int, N: int = 2, M: int = 4, out=None):
    _dev(values, meta, out)
    _flat(values, "values"), _flat(meta, "meta")
    R = values.shape[0]
    if out is None:
        out = torch.empty((R, K), dtype=values.dtype, device=values.device)
    _check(lib().nm_decompress(_dt(values), _p(values), _p(meta), R, K, N, M, _p(out), _rows(out, "out"),
                               _stream()), "nm_decompress")
    return out


def spmm_nm(values: torch.Tensor, meta: torch.Tensor, K: int, B: torch.Tensor, out=None) -> torch.Tensor:
    _dev(values, meta, B, out)
    _flat(values, "values"), _flat(meta, "meta")
    if B.dtype != values.dtype:
        raise TypeError("values and B must share a dtype")
    R = values.shape[0]
    Nc = B.shape[1]
    if B.shape[0] != K:
        raise ValueError("B must have K rows")
    if out is None:
        out = torch.empty((R, Nc), dtype=torch.float32, device=B.device)
    _check(lib().spmm_nm(_dt(B), _p(values), _p(meta), R, K, _p(B), _rows(B, "B"), Nc, _p(out),
                         _rows(out, "out"), _stream()), "spmm_nm")
    return out


def spmm_nm_t(values: torch.Tensor, meta: torch.Tensor, K: int, Bt: torch.Tensor, out=None,
              out_dtype=None) -> torch.Tensor:
    """C = decompress(values, meta) @ Bt.T with Bt [Nc, K] (rows contiguous).  C is fp32, or bf16
    (each sum rounded to nearest even: spmm_nm_t_out_bf16) when `out` is bf16 or
    out_dtype=torch.bfloat16."""
    _dev(values, meta, Bt, out)
    _flat(values, "values"), _flat(meta, "meta")
    if Bt.dtype != values.dtype:
        raise TypeError("values and Bt must share a dtype")
    R = values.shape[0]
    Nc = Bt.shape[0]
    if Bt.shape[1] != K:
        raise ValueError("Bt must have K columns")
    if out is None:
        out = torch.empty((R, Nc), dtype=out_dtype or torch.float32, device=Bt.device)
    if out.dtype == torch.bfloat16:
        _check(lib().spmm_nm_t_out_bf16(_dt(Bt), _p(values), _p(meta), R, K, _p(Bt), _rows(Bt, "Bt"), Nc, _p(out),
                                        _rows(out, "out"), _stream()), "spmm_nm_t_out_bf16")
        return out
    if out.dtype != torch.float32:
        raise TypeError("out must be fp32 or bf16")
    _check(lib().spmm_nm_t(_dt(Bt), _p(values), _p(meta), R, K, _p(Bt), _rows(Bt, "Bt"), Nc, _p(out),
                           _rows(out, "out"), _stream()), "spmm_nm_t")
    return out


def spmm_nm_t_lowrank(values: torch.Tensor, meta: torch.Tensor, K: int, Bt: torch.Tensor, U: torch.Tensor,
                      Vt: torch.Tensor, out=None, Tt=None):
    """A 2:4 weight plus a low-rank adapter, applied lazily: Tt = Bt @ Vt.T ([Nc, rank], fp32) and
    C = decompress(values, meta) @ Bt.T + U @ Tt.T ([R, Nc], fp32).  Returns (C, Tt)."""
    _dev(values, meta, Bt, U, Vt, out, Tt)
    _flat(values, "values"), _flat(meta, "meta")
    if not (Bt.dtype == values.dtype == U.dtype == Vt.dtype):
        raise TypeError("values, Bt, U and Vt must share a dtype")
    R = values.shape[0]
    Nc = Bt.shape[0]
    rank = U.shape[1]
    if Bt.shape[1] != K or Vt.shape[1] != K:
        raise ValueError("Bt and Vt must have K columns")
    if U.shape[0] != R or Vt.shape[0] != rank:
        raise ValueError("U must be [R, rank] and Vt [rank, K]")
    if out is None:
        out = torch.empty((R, Nc), dtype=torch.float32, device=Bt.device)
    if Tt is None:
        Tt = torch.empty((Nc, rank), dtype=torch.float32, device=Bt.device)
    if out.dtype != torch.float32 or Tt.dtype != torch.float32:
        raise TypeError("out and Tt must be fp32")
    if tuple(Tt.shape) != (Nc, rank) or not Tt.is_contiguous():
        raise ValueError("Tt must be a contiguous [Nc, rank] tensor")
    _check(lib().spmm_nm_t_lowrank(_dt(Bt), _p(values), _p(meta), R, K, _p(Bt), _rows(Bt, "Bt"), Nc, _p(U),
                                   _rows(U, "U"), _p(Vt), _rows(Vt, "Vt"), rank, _p(Tt), _p(out), _rows(out, "out"),
                                   _stream()), "spmm_nm_t_lowrank")
    return out, Tt


def spmm_nm_t_relu_venom(values: torch.Tensor, meta: torch.Tensor, K: int, Bt: torch.Tensor, V: int = 128, M: int = 8,
                         h_values=None, h_meta=None, h_colsel=None):
    """The up-projection C = decompress(values, meta) @ Bt.T ([R, Nc]) with its activations
    h = ReLU(bf16(C)).T ([Nc, R]) pruned to V:N:M on the way out: returns (h_values, h_meta,
    h_colsel), as prune_act_venom(h, V, M, apply_relu=True) would."""
    _dev(values, meta, Bt, h_values, h_meta, h_colsel)
    _flat(values, "values"), _flat(meta, "meta")
    if Bt.dtype != values.dtype:
        raise TypeError("values and Bt must share a dtype")
    R = values.shape[0]
    Nc = Bt.shape[0]
    if Bt.shape[1] != K:
        raise ValueError("Bt must have K columns")
    nv, mb, cb = sizes(Nc, R, 2, M, V)
    if h_values is None:
        h_values = torch.empty((Nc, nv // Nc), dtype=Bt.dtype, device=Bt.device)
    if h_meta is None:
        h_meta = torch.empty((Nc, mb // Nc), dtype=torch.uint8, device=Bt.device)
    if h_colsel is None:
        h_colsel = torch.empty((Nc // V, R // M, 4), dtype=torch.uint8, device=Bt.device)
    for t, n, name in ((h_values, nv, "h_values"), (h_meta, mb, "h_meta"), (h_colsel, cb, "h_colsel")):
        _flat(t, name)
        if t.numel() < n:
            raise ValueError(f"{name} is too small")
    _check(lib().spmm_nm_t_relu_venom(_dt(Bt), _p(values), _p(meta), R, K, _p(Bt), _rows(Bt, "Bt"), Nc, V, M,
                                      _p(h_values), _p(h_meta), _p(h_colsel), _stream()), "spmm_nm_t_relu_venom")
    return h_values, h_meta, h_colsel


def general_work_bytes(dtype: torch.dtype, R: int, K: int, N: int, M: int) -> int:
    """Bytes of work memory spmm_nm_general uses for an R x K matrix in N:M form (0: none)."""
    return int(lib().nm_general_work_bytes(NM_BF16 if dtype == torch.bfloat16 else NM_F32, R, K, N, M))


def spmm_nm_general(values: torch.Tensor, meta: torch.Tensor, K: int, N: int, M: int, Bt: torch.Tensor, out=None,
                    work="auto"):
    """C = decompress(values, meta) @ Bt.T for any N:M compressed matrix (fp32 C).  `work`: a uint8
    device tensor of at least general_work_bytes(...) bytes, None for none, or "auto" to allocate
    one with torch when the pattern uses it."""
    _dev(values, meta, Bt, out)
    _flat(values, "values"), _flat(meta, "meta")
    if Bt.dtype != values.dtype:
        raise TypeError("values and Bt must share a dtype")
    R = values.shape[0]
    Nc = Bt.shape[0]
    if Bt.shape[1] != K:
        raise ValueError("Bt must have K columns")
    if out is None:
        out = torch.empty((R, Nc), dtype=torch.float32, device=Bt.device)
    if isinstance(work, str):
        if work != "auto":
            raise ValueError("work must be a tensor, None or 'auto'")
        nbytes = general_work_bytes(values.dtype, R, K, N, M)
        work = torch.empty(nbytes, dtype=torch.uint8, device=Bt.device) if nbytes else None
    if work is not None:
        _dev(work)
        _flat(work, "work")
    _check(lib().spmm_nm_general(_dt(Bt), _p(values), _p(meta), R, K, N, M, _p(Bt), _rows(Bt, "Bt"), Nc, _p(out),
                                 _rows(out, "out"), _p(work) if work is not None else None,
                                 work.numel() * work.element_size() if work is not None else 0, _stream()),
           "spmm_nm_general")
    return out


def spmm_nm_general_noalloc(values: torch.Tensor, meta: torch.Tensor, K: int, N: int, M: int, Bt: torch.Tensor,
                            out: torch.Tensor) -> torch.Tensor:
    """spmm_nm_general with the library's fixed scratch buffer instead of work memory: the call
    allocates nothing (the caller passes `out`).  Calls that overlap on one GPU race."""
    _dev(values, meta, Bt, out)
    _flat(values, "values"), _flat(meta, "meta")
    if Bt.dtype != values.dtype:
        raise TypeError("values and Bt must share a dtype")
    R = values.shape[0]
    Nc = Bt.shape[0]
    if Bt.shape[1] != K or tuple(out.shape) != (R, Nc) or out.dtype != torch.float32:
        raise ValueError("Bt must have K columns and out must be an fp32 [R, Nc] tensor")
    _check(lib().spmm_nm_general_noalloc(_dt(Bt), _p(values), _p(meta), R, K, N, M, _p(Bt), _rows(Bt, "Bt"), Nc,
                                         _p(out), _rows(out, "out"), _stream()), "spmm_nm_general_noalloc")
    return out


def sddmm_venom(dY: torch.Tensor, W_down: torch.Tensor, h_values: torch.Tensor, h_meta: torch.Tensor,
                h_colsel: torch.Tensor, V: int, M: int = 8, apply_relu: bool = True, out=None, dYt=None):
    """dZ [T, (F/M)*2] fp32: dY @ W_down^T at the entries the V:N:M activations h_s keep (times
    ReLU's derivative when apply_relu).  With `dYt` (a [Nc, T] bf16 tensor) the call also writes
    dY^T there and returns (out, dYt)."""
    _dev(dY, W_down, h_values, h_meta, h_colsel, out, dYt)
    _flat(h_values, "h_values"), _flat(h_meta, "h_meta"), _flat(h_colsel, "h_colsel")
    if dY.dtype != W_down.dtype or h_values.dtype != dY.dtype:
        raise TypeError("dY, W_down and h_values must share a dtype")
    T, Nc = dY.shape
    F = W_down.shape[0]
    if W_down.shape[1] != Nc:
        raise ValueError("W_down must have dY's number of columns")
    if out is None:
        out = torch.empty((T, F // M * 2), dtype=torch.float32, device=dY.device)
    _flat(out, "out")
    if dYt is not None and (tuple(dYt.shape) != (Nc, T) or dYt.dtype != dY.dtype):
        raise ValueError("dYt must be [Nc, T] with dY's dtype")
    _check(lib().sddmm_venom(_dt(dY), _p(dY), _rows(dY, "dY"), _p(W_down), _rows(W_down, "W_down"), T, F, Nc, V, M,
                             _p(h_values), _p(h_meta), _p(h_colsel), int(bool(apply_relu)), _p(out), _p(dYt),
                             _rows(dYt, "dYt") if dYt is not None else 0, _stream()), "sddmm_venom")
    return (out, dYt) if dYt is not None else out


def venom_tn_work_bytes(dtype: torch.dtype, T: int, F: int) -> int:
    """Bytes of work memory spmm_venom_tn uses (0: none)."""
    return int(lib().nm_venom_tn_work_bytes(NM_BF16 if dtype == torch.bfloat16 else NM_F32, T, F))


def spmm_venom_tn(h_values: torch.Tensor, h_meta: torch.Tensor, h_colsel: torch.Tensor, F: int, V: int, M: int,
                  dYt: torch.Tensor, out=None, work="auto") -> torch.Tensor:
    """dW [F, Nc] fp32 = h_s^T @ dY for V:N:M activations h_s [T, F], given dYt = dY^T [Nc, T].
    `work`: a uint8 device tensor, None, or "auto" (allocated with torch when the call uses it)."""
    _dev(h_values, h_meta, h_colsel, dYt, out)
    _flat(h_values, "h_values"), _flat(h_meta, "h_meta"), _flat(h_colsel, "h_colsel")
    if h_values.dtype != dYt.dtype:
        raise TypeError("h_values and dYt must share a dtype")
    T = h_values.shape[0]
    Nc = dYt.shape[0]
    if dYt.shape[1] != T:
        raise ValueError("dYt must be [Nc, T]")
    if out is None:
        out = torch.empty((F, Nc), dtype=torch.float32, device=dYt.device)
    if isinstance(work, str):
        if work != "auto":
            raise ValueError("work must be a tensor, None or 'auto'")
        nbytes = venom_tn_work_bytes(h_values.dtype, T, F)
        work = torch.empty(nbytes, dtype=torch.uint8, device=dYt.device) if nbytes else None
    if work is not None:
        _dev(work)
        _flat(work, "work")
    _check(lib().spmm_venom_tn(_dt(dYt), _p(h_values), _p(h_meta), _p(h_colsel), T, F, V, M, _p(dYt),
                               _rows(dYt, "dYt"), Nc, _p(out), _rows(out, "out"),
                               _p(work) if work is not None else None,
                               work.numel() * work.element_size() if work is not None else 0, _stream()),
           "spmm_venom_tn")
    return out


def general_scratch_bytes() -> int:
    """Bytes of the fixed scratch buffer spmm_nm_general_noalloc uses on each GPU."""
    return int(lib().nm_general_scratch_bytes())


def transpose(X: torch.Tensor, out=None) -> torch.Tensor:
    """out[c, r] = X[r, c] (bf16), e.g. B [K, Nc] -> Bt [Nc, K] for spmm_nm_t."""
    _dev(X, out)
    R, C = X.shape
    if out is None:
        out = torch.empty((C, R), dtype=X.dtype, device=X.device)
    if out.shape != (C, R) or out.dtype != X.dtype:
        raise ValueError("out must be [C, R] with X's dtype")
    _check(lib().nm_transpose(_dt(X), _p(X), _rows(X, "X"), R, C, _p(out), _rows(out, "out"), _stream()),
           "nm_transpose")
    return out


def prune_act_venom(Z: torch.Tensor, V: int, M: int = 8, apply_relu: bool = False, want_mask: bool = False,
                    values=None, meta=None, colsel=None, mask=None):
    _dev(Z, values, meta, colsel, mask)
    R, K = Z.shape
    nv, mb, cb = sizes(R, K, 2, M, V)
    if values is None:
        values = torch.empty((R, nv // R), dtype=Z.dtype, device=Z.device)
    if meta is None:
        meta = torch.empty((R, mb // R), dtype=torch.uint8, device=Z.device)
    if colsel is None:
        colsel = torch.empty((R // V, K // M, 4), dtype=torch.uint8, device=Z.device)
    if want_mask and mask is None:
        mask = torch.empty((R, K), dtype=torch.uint8, device=Z.device)
    _flat(values, "values"), _flat(meta, "meta"), _flat(colsel, "colsel")
    ldm = _rows(mask, "mask") if mask is not None else 0
    _check(lib().prune_act_venom(_dt(Z), _p(Z), _rows(Z, "Z"), R, K, V, M, int(bool(apply_relu)), _p(values),
                                 _p(meta), _p(colsel), _p(mask), ldm, _stream()), "prune_act_venom")
    return (values, meta, colsel, mask) if mask is not None else (values, meta, colsel)


def spmm_venom(values: torch.Tensor, meta: torch.Tensor, colsel: torch.Tensor, K: int, V: int, M: int,
               B: torch.Tensor, out=None) -> torch.Tensor:
    _dev(values, meta, colsel, B, out)
    _flat(values, "values"), _flat(meta, "meta"), _flat(colsel, "colsel")
    if B.dtype != values.dtype:
        raise TypeError("values and B must share a dtype")
    R = values.shape[0]
    Nc = B.shape[1]
    if B.shape[0] != K:
        raise ValueError("B must have K rows")
    if out is None:
        out = torch.empty((R, Nc), dtype=torch.float32, device=B.device)
    _check(lib().spmm_venom(_dt(B), _p(values), _p(meta), _p(colsel), R, K, V, M, _p(B), _rows(B, "B"), Nc,
                            _p(out), _rows(out, "out"), _stream()), "spmm_venom")
    return out


def nm_reprune_t(values: torch.Tensor, meta: torch.Tensor, R: int, K: int, values_t=None, meta_t=None):
    _dev(values, meta, values_t, meta_t)
    _flat(values, "values"), _flat(meta, "meta")
    if values_t is None:
        values_t = torch.empty((K, R // 2), dtype=values.dtype, device=values.device)
    if meta_t is None:
        meta_t = torch.empty((K, (R + 7) // 8), dtype=torch.uint8, device=values.device)
    _check(lib().nm_reprune_t(_dt(values), _p(values), _p(meta), R, K, _p(values_t), _p(meta_t), _stream()),
           "nm_reprune_t")
    return values_t, meta_t


def nm_reprune_t_transpose(values: torch.Tensor, meta: torch.Tensor, R: int, K: int, X: torch.Tensor,
                           values_t=None, meta_t=None, Xt=None):
    """nm_reprune_t of (values, meta) and transpose of X (bf16) in one launch; returns
    (values_t, meta_t, Xt)."""
    _dev(values, meta, values_t, meta_t, X, Xt)
    _flat(values, "values"), _flat(meta, "meta")
    if values_t is None:
        values_t = torch.empty((K, R // 2), dtype=values.dtype, device=values.device)
    if meta_t is None:
        meta_t = torch.empty((K, (R + 7) // 8), dtype=torch.uint8, device=values.device)
    RX, CX = X.shape
    if Xt is None:
        Xt = torch.empty((CX, RX), dtype=X.dtype, device=X.device)
    if Xt.shape != (CX, RX) or Xt.dtype != X.dtype:
        raise ValueError("Xt must be [CX, RX] with X's dtype")
    _check(lib().nm_reprune_t_transpose(_dt(values), _p(values), _p(meta), R, K, _p(values_t), _p(meta_t), _p(X),
                                        _rows(X, "X"), RX, CX, _p(Xt), _rows(Xt, "Xt"), _stream()),
           "nm_reprune_t_transpose")
    return values_t, meta_t, Xt


def mfma_rate_probe(kind: int, iters: int, sink: torch.Tensor) -> int:
    """Launch the matrix-rate probe (kind 0 dense bf16 MFMA, 1 2:4 SMFMAC) on the current stream;
    returns the dense-equivalent flops of the launch.  `sink` is an fp32 CUDA tensor of at least
    512 * 256 elements."""
    _dev(sink)
    if sink.dtype != torch.float32 or sink.numel() < 512 * 256:
        raise ValueError("sink must be an fp32 tensor of at least 131072 elements")
    flops = _i64(0)
    _check(lib().nm_mfma_rate_probe(int(kind), int(iters), _p(sink), ctypes.byref(flops), _stream()),
           "nm_mfma_rate_probe")
    return flops.value


def nm_to_panels(values: torch.Tensor, meta: torch.Tensor, R: int, K: int, values_p=None, meta_p=None):
    """The panel layout (for spmm_nm_t_panels) of a bf16 2:4 form given row-major; returns
    (values_p, meta_p), flat buffers of the row-major sizes."""
    _dev(values, meta, values_p, meta_p)
    _flat(values, "values"), _flat(meta, "meta")
    if values_p is None:
        values_p = torch.empty((R * K // 2,), dtype=values.dtype, device=values.device)
    if meta_p is None:
        meta_p = torch.empty((R * K // 8,), dtype=torch.uint8, device=values.device)
    _check(lib().nm_to_panels(_dt(values), _p(values), _p(meta), R, K, _p(values_p), _p(meta_p), _stream()),
           "nm_to_panels")
    return values_p, meta_p


def nm_reprune_t_transpose_panels(values: torch.Tensor, meta: torch.Tensor, R: int, K: int, X: torch.Tensor,
                                  values_t=None, meta_t=None, Xt=None):
    """nm_reprune_t_transpose with the re-pruned transpose (K x R, compressed along R) in the panel
    layout; returns (values_t, meta_t, Xt), values_t and meta_t flat."""
    _dev(values, meta, values_t, meta_t, X, Xt)
    _flat(values, "values"), _flat(meta, "meta")
    if values_t is None:
        values_t = torch.empty((K * R // 2,), dtype=values.dtype, device=values.device)
    if meta_t is None:
        meta_t = torch.empty((K * R // 8,), dtype=torch.uint8, device=values.device)
    RX, CX = X.shape
    if Xt is None:
        Xt = torch.empty((CX, RX), dtype=X.dtype, device=X.device)
    if Xt.shape != (CX, RX) or Xt.dtype != X.dtype:
        raise ValueError("Xt must be [CX, RX] with X's dtype")
    _check(lib().nm_reprune_t_transpose_panels(_dt(values), _p(values), _p(meta), R, K, _p(values_t), _p(meta_t),
                                               _p(X), _rows(X, "X"), RX, CX, _p(Xt), _rows(Xt, "Xt"), _stream()),
           "nm_reprune_t_transpose_panels")
    return values_t, meta_t, Xt


def spmm_nm_t_panels(values: torch.Tensor, meta: torch.Tensor, R: int, K: int, Bt: torch.Tensor, out=None):
    """spmm_nm_t of an R x K bf16 2:4 weight in the panel layout: C [R, Nc] fp32."""
    _dev(values, meta, Bt, out)
    _flat(values, "values"), _flat(meta, "meta")
    Nc = Bt.shape[0]
    if out is None:
        out = torch.empty((R, Nc), dtype=torch.float32, device=Bt.device)
    _check(lib().spmm_nm_t_panels(_dt(Bt), _p(values), _p(meta), R, K, _p(Bt), _rows(Bt, "Bt"), Nc, _p(out),
                                  _rows(out, "out"), _stream()), "spmm_nm_t_panels")
    return out


def sddmm_nm(D: torch.Tensor, X: torch.Tensor, meta: torch.Tensor, out=None, Dt=None):
    """dW values of a 2:4 layer; with `Dt` (a [T, R] tensor, bf16) the call is sddmm_nm_dt, which also
    writes Dt = D^T, and returns (out, Dt)."""
    _dev(D, X, meta, out, Dt)
    _flat(meta, "meta")
    if D.dtype != X.dtype:
        raise TypeError("D and X must share a dtype")
    R, T = D.shape
    Kc = X.shape[0]
    if X.shape[1] != T:
        raise ValueError("D and X must have the same number of columns")
    if out is None:
        out = torch.empty((R, Kc // 2), dtype=torch.float32, device=D.device)
    _flat(out, "out")
    if Dt is not None:
        if Dt.shape != (T, R) or Dt.dtype != D.dtype:
            raise ValueError("Dt must be [T, R] with D's dtype")
        _check(lib().sddmm_nm_dt(_dt(D), _p(D), _rows(D, "D"), _p(X), _rows(X, "X"), R, Kc, T, _p(meta), _p(out),
                                 _p(Dt), _rows(Dt, "Dt"), _stream()), "sddmm_nm_dt")
        return out, Dt
    _check(lib().sddmm_nm(_dt(D), _p(D), _rows(D, "D"), _p(X), _rows(X, "X"), R, Kc, T, _p(meta), _p(out),
                          _stream()), "sddmm_nm")
    return out
