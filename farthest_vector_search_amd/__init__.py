"""Python binding of libvs (masked arg-reduction scans on MI355X / gfx950).

Argument marshalling only: every step of every search runs in the HIP
kernels of ``libvs.so``, called through its C ABI (``include/vs.h``) on the
current torch stream.  PyTorch supplies device memory and streams.  There is
no CPU fallback: if the library is missing or no gfx950 GPU is present the
calls raise.

Functions (same names as the C entry points):
    vs_bmu_search(Q, C, metric)                        -> (idx, score)
    vs_bmu_search_noalloc(Q, C, metric)                -> (idx, score), no workspace
    vs_bmu_search_unfused(Q, C, metric)                -> (idx, score) via a score block
    vs_bmu_search_csr(indptr, indices, values, CT, metric) -> (idx, score)
    vs_csr_block_codebook(CT)                          -> CB (64-neuron blocked copy)
    vs_bmu_search_csr_blocked(indptr, indices, values, CB, nc, metric) -> (idx, score)
    vs_csr_block_codebook_f16(CT)                      -> CB16 (fp16, 128-neuron blocks)
    vs_bmu_search_csr_blocked_f16(indptr, indices, values, CB16, nc, metric) -> (idx, score)
    vs_diversity_step(C, last_pick, mask_bits)         -> (idx, score)
    vs_diversity_gram(C)                               -> G (n x ldg Gram matrix)
    vs_diversity_step_gram(G, n, last_pick, mask_bits) -> (idx, score)
    vs_candidate_norms(C, feature_major=False)         -> norms
    vs_tile_rows(cache_bytes, d, bytes_per_value)      -> int (host only)
Metrics: VS_L2SQ_MIN, VS_L2SQ_MAX, VS_COS_MAX, VS_COS_MIN.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvs.so")

VS_L2SQ_MIN, VS_L2SQ_MAX, VS_COS_MAX, VS_COS_MIN = 0, 1, 2, 3
METRICS = {"l2sq_min": 0, "l2sq_max": 1, "cos_max": 2, "cos_min": 3}

STATUS = {0: "VS_OK", 1: "VS_ERR_NULL", 2: "VS_ERR_SHAPE", 3: "VS_ERR_METRIC",
          4: "VS_ERR_WORKSPACE", 5: "VS_ERR_ALIGN", 6: "VS_ERR_INDEX",
          7: "VS_ERR_UNSUPPORTED", 8: "VS_ERR_HIP"}

EXPORTS = ["vs_bmu_search_workspace", "vs_bmu_search", "vs_bmu_search_noalloc",
           "vs_bmu_search_unfused",
           "vs_bmu_search_csr_workspace",
           "vs_bmu_search_csr", "vs_csr_blocked_bytes", "vs_csr_block_codebook",
           "vs_bmu_search_csr_blocked", "vs_csr_blocked_f16_bytes", "vs_csr_block_codebook_f16",
           "vs_bmu_search_csr_blocked_f16", "vs_diversity_step_workspace", "vs_diversity_step",
           "vs_diversity_run", "vs_diversity_run_gram", "vs_diversity_run_ref",
           "vs_diversity_step_ref", "vs_diversity_accumulate",
           "vs_diversity_gram", "vs_diversity_step_gram", "vs_diversity_step_gram_sum",
           "vs_som_update_workspace", "vs_som_update", "vs_som_update_csr", "vs_som_qe",
           "vs_som_epoch_workspace", "vs_som_epoch", "vs_som_epoch_csr_workspace",
           "vs_som_epoch_csr", "vs_som_epoch_csr_f16", "vs_csr_blocked_to_f16",
           "vs_candidate_norms", "vs_tile_rows", "vs_timing_enable", "vs_timing_read",
           "vs_timing_kernel_name", "vs_status_str", "vs_last_hip_error", "vs_version"]


class VsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)}"
        if status == 8 and _lib is not None:
            msg += f" (hip error {_lib.vs_last_hip_error()})"
        super().__init__(msg)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libvs.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m farthest_vector_search_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.vs_bmu_search_workspace.argtypes = [I64, I64, I32, I32]
    L.vs_bmu_search_workspace.restype = SZ
    L.vs_bmu_search.argtypes = [P, P, I64, I64, I32, I32, P, P, P, SZ, P]
    L.vs_bmu_search_noalloc.argtypes = [P, P, I64, I64, I32, I32, P, P, P]
    L.vs_bmu_search_unfused.argtypes = [P, P, I64, I64, I32, I32, P, P, P, I64, P, SZ, P]
    L.vs_bmu_search_csr_workspace.argtypes = [I64, I64, I32, I32]
    L.vs_bmu_search_csr_workspace.restype = SZ
    L.vs_bmu_search_csr.argtypes = [P, P, P, I64, I64, P, I64, I64, I32, I32, P, P, P, SZ, P]
    L.vs_csr_blocked_bytes.argtypes = [I64, I32]
    L.vs_csr_blocked_bytes.restype = SZ
    L.vs_csr_block_codebook.argtypes = [P, I64, I64, I32, P, P]
    L.vs_bmu_search_csr_blocked.argtypes = [P, P, P, I64, I64, P, I64, I32, I32, P, P, P, SZ, P]
    L.vs_csr_blocked_f16_bytes.argtypes = [I64, I32]
    L.vs_csr_blocked_f16_bytes.restype = SZ
    L.vs_csr_block_codebook_f16.argtypes = [P, I64, I64, I32, P, P]
    L.vs_bmu_search_csr_blocked_f16.argtypes = [P, P, P, I64, I64, P, I64, I32, I32, P, P, P, SZ,
                                                P]
    L.vs_diversity_step_workspace.argtypes = [I64, I32, I64]
    L.vs_diversity_step_workspace.restype = SZ
    L.vs_diversity_step.argtypes = [P, I64, I32, P, P, I64, P, P, P, SZ, P]
    L.vs_diversity_step_ref.argtypes = [P, I64, I32, P, P, I64, P, P, P, SZ, P]
    L.vs_diversity_accumulate.argtypes = [P, I64, I32, P, P, I64, P]
    L.vs_diversity_gram.argtypes = [P, I64, I32, P, I64, P]
    L.vs_diversity_step_gram.argtypes = [P, I64, I64, P, P, I64, P, P, P]
    L.vs_diversity_step_gram_sum.argtypes = [P, I64, I64, P, P, I64, P, I64, P, P, P]
    L.vs_diversity_run.argtypes = [P, I64, I32, P, P, I64, I32, P, P, P, SZ, P]
    L.vs_diversity_run_gram.argtypes = [P, I64, I64, P, P, I64, P, I64, I32, P, P, P]
    L.vs_diversity_run_ref.argtypes = [P, I64, I32, P, P, P, I64, I32, P, P, P, SZ, P]
    F = ctypes.c_float
    L.vs_som_update_workspace.argtypes = [I32, I32, I32]
    L.vs_som_update_workspace.restype = SZ
    L.vs_som_update.argtypes = [P, I64, I32, P, P, I32, I32, F, I32, P, SZ, P]
    L.vs_som_update_csr.argtypes = [P, P, P, I64, I64, P, P, I32, I32, I32, F, I32, P, SZ, P]
    L.vs_som_qe.argtypes = [P, I64, P, P]
    L.vs_som_epoch_workspace.argtypes = [I64, I32, I32, I32]
    L.vs_som_epoch_workspace.restype = SZ
    L.vs_som_epoch.argtypes = [P, I64, I32, P, I32, I32, F, I32, P, P, P, P, SZ, P]
    L.vs_som_epoch_csr_workspace.argtypes = [I64, I32, I32, I32]
    L.vs_som_epoch_csr_workspace.restype = SZ
    L.vs_som_epoch_csr.argtypes = [P, P, P, I64, I64, P, I32, I32, I32, F, I32, P, P, P, P, SZ,
                                   P]
    L.vs_csr_blocked_to_f16.argtypes = [P, I64, I32, P, P]
    L.vs_som_epoch_csr_f16.argtypes = [P, P, P, I64, I64, P, P, I32, I32, I32, F, I32, P, P, P,
                                       P, SZ, P]
    L.vs_candidate_norms.argtypes = [P, I64, I32, I32, P, P]
    L.vs_tile_rows.argtypes = [I64, I32, I32]
    L.vs_tile_rows.restype = I64
    L.vs_timing_enable.argtypes = [I32]
    L.vs_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)]
    L.vs_timing_kernel_name.restype = ctypes.c_char_p
    L.vs_status_str.argtypes = [ctypes.c_int]
    L.vs_status_str.restype = ctypes.c_char_p
    L.vs_version.restype = ctypes.c_char_p
    for name in ("vs_bmu_search", "vs_bmu_search_noalloc", "vs_bmu_search_unfused",
                 "vs_bmu_search_csr",
                 "vs_csr_block_codebook",
                 "vs_bmu_search_csr_blocked", "vs_csr_block_codebook_f16",
                 "vs_bmu_search_csr_blocked_f16", "vs_diversity_step", "vs_diversity_gram",
                 "vs_diversity_step_gram", "vs_diversity_step_ref", "vs_diversity_accumulate",
                 "vs_diversity_step_gram_sum", "vs_diversity_run", "vs_diversity_run_gram",
                 "vs_diversity_run_ref",
                 "vs_som_update", "vs_som_update_csr", "vs_som_qe",
                 "vs_som_epoch", "vs_som_epoch_csr", "vs_som_epoch_csr_f16",
                 "vs_csr_blocked_to_f16",
                 "vs_candidate_norms", "vs_timing_enable", "vs_timing_read",
                 "vs_last_hip_error"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


# ---------------------------------------------------------------- helpers --

def _torch():
    import torch
    return torch


def _metric(m) -> int:
    return METRICS[m] if isinstance(m, str) else int(m)


def _dev(t, name, dtype, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


_raw_stream = None


def _stream(device):
    """The raw handle of torch's current stream on `device` (the call's
    stream).  torch's own raw-handle accessor where present: the public
    Stream object costs a few microseconds per call."""
    global _raw_stream
    torch = _torch()
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    i = device.index if device.index is not None else torch.cuda.current_device()
    if _raw_stream:
        return _raw_stream(i)
    return torch.cuda.current_stream(i).cuda_stream


_same_device = contextlib.nullcontext()
_get_device = None


def _on(device):
    """Make `device` current for the call (a no-op when it already is)."""
    global _get_device
    torch = _torch()
    if _get_device is None:
        _get_device = getattr(torch._C, "_cuda_getDevice", torch.cuda.current_device)
    if device.index is None or device.index == _get_device():
        return _same_device
    return torch.cuda.device(device)


def _check(rc: int, where: str):
    if rc != 0:
        raise VsError(rc, where)


def _out(t, name, dtype, shape, device, want: bool = True):
    """A caller's output tensor, checked (device, dtype, contiguity, at least
    the elements the call writes), or a new one; None when not wanted."""
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device) if want else None
    _dev(t, name, dtype)
    if t.device != (device if isinstance(device, torch.device) else torch.device(device)):
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    n = 1
    for v in (shape if isinstance(shape, tuple) else (shape,)):
        n *= max(int(v), 0)
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the call writes {n}")
    return t


def _workspace(nbytes: int, device, workspace):
    torch = _torch()
    if workspace is None:
        return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise TypeError("workspace must be a CUDA (HIP) torch tensor")
    if workspace.device != (device if isinstance(device, torch.device) else torch.device(device)):
        raise ValueError(f"workspace is on {workspace.device}, the inputs on {device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace too small")
    return workspace


# ------------------------------------------------------------ entry points --

def vs_bmu_search(Q, C, metric=VS_L2SQ_MIN, idx_out=None, score_out=None, workspace=None,
                  want_score: bool = True):
    """Best candidate row of C for every row of Q (see include/vs.h)."""
    torch = _torch()
    L = lib()
    m = _metric(metric)
    _dev(Q, "Q", torch.float32, 2)
    _dev(C, "C", torch.float32, 2)
    nq, d = Q.shape
    nc = C.shape[0]
    if C.shape[1] != d:
        raise ValueError("Q and C must have the same number of columns")
    dev = Q.device
    idx_out = _out(idx_out, "idx_out", torch.int32, nq, dev)
    score_out = _out(score_out, "score_out", torch.float32, nq, dev, want_score)
    need = L.vs_bmu_search_workspace(nq, nc, d, m)
    ws = _workspace(need, dev, workspace)
    with _on(dev):
        rc = L.vs_bmu_search(_ptr(Q), _ptr(C), nq, nc, d, m, _ptr(idx_out), _ptr(score_out),
                             _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_bmu_search")
    return idx_out, score_out


def vs_bmu_search_noalloc(Q, C, metric=VS_L2SQ_MIN, idx_out=None, score_out=None,
                          want_score: bool = True):
    """vs_bmu_search without a workspace: the library's own device scratch
    array serves as one (at most 8 MiB of workspace; calls that overlap on
    one GPU race).  Pass idx_out / score_out to make the call allocate
    nothing at all."""
    torch = _torch()
    L = lib()
    m = _metric(metric)
    _dev(Q, "Q", torch.float32, 2)
    _dev(C, "C", torch.float32, 2)
    nq, d = Q.shape
    nc = C.shape[0]
    if C.shape[1] != d:
        raise ValueError("Q and C must have the same number of columns")
    dev = Q.device
    idx_out = _out(idx_out, "idx_out", torch.int32, nq, dev)
    score_out = _out(score_out, "score_out", torch.float32, nq, dev, want_score)
    with _on(dev):
        rc = L.vs_bmu_search_noalloc(_ptr(Q), _ptr(C), nq, nc, d, m, _ptr(idx_out),
                                     _ptr(score_out), _stream(dev))
    _check(rc, "vs_bmu_search_noalloc")
    return idx_out, score_out


def vs_bmu_search_unfused(Q, C, metric=VS_L2SQ_MIN, S=None, idx_out=None, score_out=None,
                          workspace=None, want_score: bool = True):
    """vs_bmu_search through a written score block S (nq x ld_s float32, the
    unfused comparator; allocated here if not given)."""
    torch = _torch()
    L = lib()
    m = _metric(metric)
    _dev(Q, "Q", torch.float32, 2)
    _dev(C, "C", torch.float32, 2)
    nq, d = Q.shape
    nc = C.shape[0]
    if C.shape[1] != d:
        raise ValueError("Q and C must have the same number of columns")
    dev = Q.device
    if S is None:
        S = torch.empty((nq, (nc + 63) // 64 * 64), dtype=torch.float32, device=dev)
    elif not isinstance(S, torch.Tensor) or not S.is_cuda or S.device != dev \
            or S.dtype != torch.float32 or S.dim() != 2 or S.shape[0] < nq or S.shape[1] < nc \
            or S.stride(1) != 1 or S.stride(0) % 4:
        raise ValueError("S must be a float32 nq x ld_s matrix (ld_s >= nc, ld_s % 4 == 0) "
                         "on the device of Q")
    idx_out = _out(idx_out, "idx_out", torch.int32, nq, dev)
    score_out = _out(score_out, "score_out", torch.float32, nq, dev, want_score)
    need = L.vs_bmu_search_workspace(nq, nc, d, m)
    ws = _workspace(need, dev, workspace)
    with _on(dev):
        rc = L.vs_bmu_search_unfused(_ptr(Q), _ptr(C), nq, nc, d, m, _ptr(idx_out),
                                     _ptr(score_out), _ptr(S), S.stride(0), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_bmu_search_unfused")
    return idx_out, score_out


def vs_bmu_search_csr(indptr, indices, values, CT, metric=VS_L2SQ_MIN, idx_out=None,
                      score_out=None, workspace=None, want_score: bool = True):
    """Best codebook column of CT (d x nc, feature-major) for every CSR row.

    CT may be a row-padded view (CT.stride(0) > nc), e.g.
    ``torch.empty(d, nc + 64)[:, :nc]``: its row stride is passed as ldct."""
    torch = _torch()
    L = lib()
    m = _metric(metric)
    _dev(indptr, "indptr", torch.int32, 1)
    _dev(indices, "indices", torch.int32, 1)
    _dev(values, "values", torch.float32, 1)
    if not isinstance(CT, torch.Tensor) or not CT.is_cuda or CT.dtype != torch.float32 \
            or CT.dim() != 2 or CT.stride(1) != 1 or CT.stride(0) < CT.shape[1]:
        raise ValueError("CT must be a float32 CUDA matrix with unit column stride")
    nq = indptr.numel() - 1
    nnz = indices.numel()
    if values.numel() != nnz:
        raise ValueError("indices and values differ in length")
    d, nc = CT.shape
    dev = CT.device
    idx_out = _out(idx_out, "idx_out", torch.int32, max(nq, 0), dev)
    score_out = _out(score_out, "score_out", torch.float32, max(nq, 0), dev, want_score)
    need = L.vs_bmu_search_csr_workspace(nq, nc, d, m)
    ws = _workspace(need, dev, workspace)
    with _on(dev):
        rc = L.vs_bmu_search_csr(_ptr(indptr), _ptr(indices) if nnz else None,
                                 _ptr(values) if nnz else None, nq, nnz, _ptr(CT), nc,
                                 CT.stride(0), d, m,
                                 _ptr(idx_out), _ptr(score_out), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_bmu_search_csr")
    return idx_out, score_out


def vs_csr_block_codebook(CT, out=None):
    """64-neuron blocked copy of a feature-major codebook CT (d x nc, unit
    column stride, any row stride): a flat float32 tensor holding, for every
    block b, the d x 64 matrix of neurons 64 b .. 64 b + 63 (zeros past nc)."""
    torch = _torch()
    L = lib()
    if not isinstance(CT, torch.Tensor) or not CT.is_cuda or CT.dtype != torch.float32 \
            or CT.dim() != 2 or CT.stride(1) != 1 or CT.stride(0) < CT.shape[1]:
        raise ValueError("CT must be a float32 CUDA matrix with unit column stride")
    d, nc = CT.shape
    n = L.vs_csr_blocked_bytes(nc, d) // 4
    out = _out(out, "out", torch.float32, n, CT.device)
    with _on(CT.device):
        rc = L.vs_csr_block_codebook(_ptr(CT), nc, CT.stride(0), d, _ptr(out),
                                     _stream(CT.device))
    _check(rc, "vs_csr_block_codebook")
    return out


def vs_bmu_search_csr_blocked(indptr, indices, values, CB, nc, metric=VS_L2SQ_MIN, d=None,
                              idx_out=None, score_out=None, workspace=None,
                              want_score: bool = True):
    """vs_bmu_search_csr over a codebook in the 64-neuron blocked layout that
    vs_csr_block_codebook writes (nc neurons, d features)."""
    torch = _torch()
    L = lib()
    m = _metric(metric)
    _dev(indptr, "indptr", torch.int32, 1)
    _dev(indices, "indices", torch.int32, 1)
    _dev(values, "values", torch.float32, 1)
    _dev(CB, "CB", torch.float32, 1)
    nq = indptr.numel() - 1
    nnz = indices.numel()
    if values.numel() != nnz:
        raise ValueError("indices and values differ in length")
    nblk = (nc + 63) // 64
    if d is None:
        d = CB.numel() // (nblk * 64)
    if CB.numel() < nblk * 64 * d:
        raise ValueError("CB is smaller than the blocked layout of nc x d")
    dev = CB.device
    idx_out = _out(idx_out, "idx_out", torch.int32, max(nq, 0), dev)
    score_out = _out(score_out, "score_out", torch.float32, max(nq, 0), dev, want_score)
    need = L.vs_bmu_search_csr_workspace(nq, nc, d, m)
    ws = _workspace(need, dev, workspace)
    with _on(dev):
        rc = L.vs_bmu_search_csr_blocked(_ptr(indptr), _ptr(indices) if nnz else None,
                                         _ptr(values) if nnz else None, nq, nnz, _ptr(CB), nc,
                                         d, m, _ptr(idx_out), _ptr(score_out), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_bmu_search_csr_blocked")
    return idx_out, score_out


def vs_csr_block_codebook_f16(CT, out=None):
    """fp16 copy of a feature-major fp32 codebook CT (d x nc, unit column
    stride, any row stride) in 128-neuron blocks: a flat torch.float16 tensor
    holding, for every block b, the d x 128 matrix of neurons 128 b ..
    128 b + 127 (zeros past nc), rounded to nearest even."""
    torch = _torch()
    L = lib()
    if not isinstance(CT, torch.Tensor) or not CT.is_cuda or CT.dtype != torch.float32 \
            or CT.dim() != 2 or CT.stride(1) != 1 or CT.stride(0) < CT.shape[1]:
        raise ValueError("CT must be a float32 CUDA matrix with unit column stride")
    d, nc = CT.shape
    n = L.vs_csr_blocked_f16_bytes(nc, d) // 2
    out = _out(out, "out", torch.float16, n, CT.device)
    with _on(CT.device):
        rc = L.vs_csr_block_codebook_f16(_ptr(CT), nc, CT.stride(0), d, _ptr(out),
                                         _stream(CT.device))
    _check(rc, "vs_csr_block_codebook_f16")
    return out


def vs_bmu_search_csr_blocked_f16(indptr, indices, values, CB16, nc, metric=VS_L2SQ_MIN, d=None,
                                  idx_out=None, score_out=None, workspace=None,
                                  want_score: bool = True):
    """vs_bmu_search_csr over an fp16 codebook in the 128-neuron blocked layout
    that vs_csr_block_codebook_f16 writes (fp32 arithmetic throughout)."""
    torch = _torch()
    L = lib()
    m = _metric(metric)
    _dev(indptr, "indptr", torch.int32, 1)
    _dev(indices, "indices", torch.int32, 1)
    _dev(values, "values", torch.float32, 1)
    _dev(CB16, "CB16", torch.float16, 1)
    nq = indptr.numel() - 1
    nnz = indices.numel()
    if values.numel() != nnz:
        raise ValueError("indices and values differ in length")
    nblk = (nc + 127) // 128
    if d is None:
        d = CB16.numel() // (nblk * 128)
    if CB16.numel() < nblk * 128 * d:
        raise ValueError("CB16 is smaller than the blocked layout of nc x d")
    dev = CB16.device
    idx_out = _out(idx_out, "idx_out", torch.int32, max(nq, 0), dev)
    score_out = _out(score_out, "score_out", torch.float32, max(nq, 0), dev, want_score)
    need = L.vs_bmu_search_csr_workspace(nq, nc, d, m)
    ws = _workspace(need, dev, workspace)
    with _on(dev):
        rc = L.vs_bmu_search_csr_blocked_f16(_ptr(indptr), _ptr(indices) if nnz else None,
                                             _ptr(values) if nnz else None, nq, nnz, _ptr(CB16),
                                             nc, d, m, _ptr(idx_out), _ptr(score_out), _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_bmu_search_csr_blocked_f16")
    return idx_out, score_out


def vs_diversity_step(C, last_pick, mask_bits, idx_out=None, score_out=None, workspace=None,
                      want_score: bool = True):
    """One greedy diversity step for every sequence; updates mask_bits in place."""
    torch = _torch()
    L = lib()
    _dev(C, "C", torch.float32, 2)
    _dev(last_pick, "last_pick", torch.int32, 1)
    n, d = C.shape
    nseq = last_pick.numel()
    W = (n + 31) // 32
    if mask_bits.dtype not in (torch.int32, torch.uint32):
        raise TypeError("mask_bits must be int32 or uint32 words")
    _dev(mask_bits, "mask_bits", mask_bits.dtype, 2)
    if tuple(mask_bits.shape) != (nseq, W):
        raise ValueError(f"mask_bits must be [{nseq}, {W}]")
    dev = C.device
    idx_out = _out(idx_out, "idx_out", torch.int32, nseq, dev)
    score_out = _out(score_out, "score_out", torch.float32, nseq, dev, want_score)
    need = L.vs_diversity_step_workspace(n, d, nseq)
    ws = _workspace(need, dev, workspace)
    with _on(dev):
        rc = L.vs_diversity_step(_ptr(C), n, d, _ptr(last_pick), _ptr(mask_bits), nseq,
                                 _ptr(idx_out), _ptr(score_out), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_diversity_step")
    return idx_out, score_out


def vs_diversity_step_ref(C, Q, mask_bits, idx_out=None, score_out=None, workspace=None,
                          want_score: bool = True):
    """One diversity step against explicit reference rows Q (nseq x d)."""
    torch = _torch()
    L = lib()
    _dev(C, "C", torch.float32, 2)
    _dev(Q, "Q", torch.float32, 2)
    if mask_bits.dtype not in (torch.int32, torch.uint32):
        raise TypeError("mask_bits must be int32 or uint32 words")
    _dev(mask_bits, "mask_bits", mask_bits.dtype, 2)
    n, d = C.shape
    nseq = Q.shape[0]
    if Q.shape[1] != d or tuple(mask_bits.shape) != (nseq, mask_words(n)):
        raise ValueError("Q or mask_bits disagree with C")
    dev = C.device
    idx_out = _out(idx_out, "idx_out", torch.int32, nseq, dev)
    score_out = _out(score_out, "score_out", torch.float32, nseq, dev, want_score)
    ws = _workspace(L.vs_diversity_step_workspace(n, d, nseq), dev, workspace)
    with _on(dev):
        rc = L.vs_diversity_step_ref(_ptr(C), n, d, _ptr(Q), _ptr(mask_bits), nseq,
                                     _ptr(idx_out), _ptr(score_out), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_diversity_step_ref")
    return idx_out, score_out


def vs_diversity_accumulate(C, pick, Q):
    """Q[s] += C[pick[s]] where the pick is valid (in place)."""
    torch = _torch()
    L = lib()
    _dev(C, "C", torch.float32, 2)
    _dev(pick, "pick", torch.int32, 1)
    _dev(Q, "Q", torch.float32, 2)
    n, d = C.shape
    if Q.shape != (pick.numel(), d):
        raise ValueError("Q must be (len(pick), d)")
    with _on(C.device):
        rc = L.vs_diversity_accumulate(_ptr(C), n, d, _ptr(pick), _ptr(Q), pick.numel(),
                                       _stream(C.device))
    _check(rc, "vs_diversity_accumulate")
    return Q


def vs_diversity_gram(C, out=None):
    """Gram matrix of the table C (n x d, unit rows) by the diversity step's
    own arithmetic: returns G, an n x ldg float32 view (ldg = n rounded up to
    a multiple of 64) whose entry [r, j] is C[r] . C[j]."""
    torch = _torch()
    L = lib()
    _dev(C, "C", torch.float32, 2)
    n, d = C.shape
    ldg = (n + 63) // 64 * 64
    if out is None:
        out = torch.empty((n, ldg), dtype=torch.float32, device=C.device)
    elif not out.is_cuda or out.device != C.device or out.dtype != torch.float32 \
            or out.dim() != 2 or out.shape[0] != n or out.shape[1] < n or out.stride(1) != 1 \
            or out.stride(0) % 4:
        raise ValueError("out must be a float32 n x ldg matrix (ldg >= n, ldg % 4 == 0) "
                         "on the device of C")
    with _on(C.device):
        rc = L.vs_diversity_gram(_ptr(C), n, d, _ptr(out), out.stride(0), _stream(C.device))
    _check(rc, "vs_diversity_gram")
    return out[:, :n]


def vs_diversity_step_gram(G, last_pick, mask_bits, idx_out=None, score_out=None,
                           want_score: bool = True):
    """One diversity step for every sequence from a cached Gram matrix G (a
    view returned by vs_diversity_gram); updates mask_bits in place."""
    torch = _torch()
    L = lib()
    if not isinstance(G, torch.Tensor) or not G.is_cuda or G.dtype != torch.float32 \
            or G.dim() != 2 or G.stride(1) != 1 or G.shape[0] != G.shape[1]:
        raise ValueError("G must be a square float32 CUDA matrix view with unit column stride")
    _dev(last_pick, "last_pick", torch.int32, 1)
    n = G.shape[0]
    nseq = last_pick.numel()
    W = (n + 31) // 32
    if mask_bits.dtype not in (torch.int32, torch.uint32):
        raise TypeError("mask_bits must be int32 or uint32 words")
    _dev(mask_bits, "mask_bits", mask_bits.dtype, 2)
    if tuple(mask_bits.shape) != (nseq, W):
        raise ValueError(f"mask_bits must be [{nseq}, {W}]")
    dev = G.device
    idx_out = _out(idx_out, "idx_out", torch.int32, nseq, dev)
    score_out = _out(score_out, "score_out", torch.float32, nseq, dev, want_score)
    with _on(dev):
        rc = L.vs_diversity_step_gram(_ptr(G), n, G.stride(0), _ptr(last_pick), _ptr(mask_bits),
                                      nseq, _ptr(idx_out), _ptr(score_out), _stream(dev))
    _check(rc, "vs_diversity_step_gram")
    return idx_out, score_out


def _mask_arg(mask_bits, nseq, n):
    torch = _torch()
    if mask_bits.dtype not in (torch.int32, torch.uint32):
        raise TypeError("mask_bits must be int32 or uint32 words")
    _dev(mask_bits, "mask_bits", mask_bits.dtype, 2)
    if tuple(mask_bits.shape) != (nseq, (n + 31) // 32):
        raise ValueError(f"mask_bits must be [{nseq}, {(n + 31) // 32}]")


def vs_diversity_run(C, seeds, mask_bits, steps: int, picks_out=None, scores_out=None,
                     workspace=None, want_scores: bool = True):
    """`steps` diversity steps from the seeds; returns picks [steps, nseq] and
    scores [steps, nseq] (or None).  mask_bits (seed bits set) is updated."""
    torch = _torch()
    L = lib()
    _dev(C, "C", torch.float32, 2)
    _dev(seeds, "seeds", torch.int32, 1)
    n, d = C.shape
    nseq = seeds.numel()
    _mask_arg(mask_bits, nseq, n)
    dev = C.device
    picks_out = _out(picks_out, "picks_out", torch.int32, (steps, nseq), dev)
    scores_out = _out(scores_out, "scores_out", torch.float32, (steps, nseq), dev, want_scores)
    ws = _workspace(L.vs_diversity_step_workspace(n, d, nseq), dev, workspace)
    with _on(dev):
        rc = L.vs_diversity_run(_ptr(C), n, d, _ptr(seeds), _ptr(mask_bits), nseq, int(steps),
                                _ptr(picks_out), _ptr(scores_out), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_diversity_run")
    return picks_out, scores_out


def vs_diversity_run_ref(C, seeds, mask_bits, steps: int, Q=None, picks_out=None,
                         scores_out=None, workspace=None, want_scores: bool = True):
    """A whole centroid-reading run with explicit references; returns (picks,
    scores, Q) with Q the final per-sequence sums of rows."""
    torch = _torch()
    L = lib()
    _dev(C, "C", torch.float32, 2)
    _dev(seeds, "seeds", torch.int32, 1)
    n, d = C.shape
    nseq = seeds.numel()
    _mask_arg(mask_bits, nseq, n)
    dev = C.device
    Q = _out(Q, "Q", torch.float32, (nseq, d), dev)
    _dev(Q, "Q", torch.float32, 2)
    if tuple(Q.shape) != (nseq, d):
        raise ValueError("Q must be (nseq, d)")
    picks_out = _out(picks_out, "picks_out", torch.int32, (steps, nseq), dev)
    scores_out = _out(scores_out, "scores_out", torch.float32, (steps, nseq), dev, want_scores)
    ws = _workspace(L.vs_diversity_step_workspace(n, d, nseq), dev, workspace)
    with _on(dev):
        rc = L.vs_diversity_run_ref(_ptr(C), n, d, _ptr(seeds), _ptr(Q), _ptr(mask_bits), nseq,
                                    int(steps), _ptr(picks_out), _ptr(scores_out), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_diversity_run_ref")
    return picks_out, scores_out, Q


def vs_diversity_run_gram(G, seeds, mask_bits, steps: int, R=None, picks_out=None,
                          scores_out=None, want_scores: bool = True):
    """A whole run from the Gram matrix G: the last-pick reading, or with R
    (rows from vs_diversity_gram_sums; cleared by the call) the centroid one."""
    torch = _torch()
    L = lib()
    for name, t in (("G", G), ("R", R)):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 \
                or t.dim() != 2 or t.stride(1) != 1 or t.device != G.device:
            raise ValueError(f"{name} must be a float32 CUDA matrix view with unit column stride"
                             " on the device of G")
    _dev(seeds, "seeds", torch.int32, 1)
    n = G.shape[0]
    nseq = seeds.numel()
    if G.shape[1] != n or (R is not None and tuple(R.shape) != (nseq, n)):
        raise ValueError("G must be n x n and R nseq x n")
    _mask_arg(mask_bits, nseq, n)
    dev = G.device
    picks_out = _out(picks_out, "picks_out", torch.int32, (steps, nseq), dev)
    scores_out = _out(scores_out, "scores_out", torch.float32, (steps, nseq), dev, want_scores)
    with _on(dev):
        rc = L.vs_diversity_run_gram(_ptr(G), n, G.stride(0), _ptr(seeds), _ptr(R),
                                     0 if R is None else R.stride(0), _ptr(mask_bits), nseq,
                                     int(steps), _ptr(picks_out), _ptr(scores_out), _stream(dev))
    _check(rc, "vs_diversity_run_gram")
    return picks_out, scores_out


def vs_diversity_gram_sums(G, nseq: int, out=None):
    """Zeroed running-sum rows R for vs_diversity_step_gram_sum: an
    (nseq, n) view of an (nseq, ldr) float32 buffer, ldr = n rounded up to 64."""
    torch = _torch()
    n = G.shape[0]
    ldr = (n + 63) // 64 * 64
    out = _out(out, "out", torch.float32, (nseq, ldr), G.device).view(-1)[:nseq * ldr]
    out = out.view(nseq, ldr)
    out.zero_()
    return out[:, :n]


def vs_diversity_step_gram_sum(G, last_pick, R, mask_bits, idx_out=None, score_out=None,
                               want_score: bool = True):
    """One centroid-reference step from the Gram matrix: R[s] += G[last_pick[s]],
    then the masked arg-min of R[s] (R from vs_diversity_gram_sums, updated
    in place, as is mask_bits)."""
    torch = _torch()
    L = lib()
    for name, t in (("G", G), ("R", R)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 \
                or t.dim() != 2 or t.stride(1) != 1 or t.device != G.device:
            raise ValueError(f"{name} must be a float32 CUDA matrix view with unit column stride"
                             " on the device of G")
    _dev(last_pick, "last_pick", torch.int32, 1)
    n = G.shape[0]
    nseq = last_pick.numel()
    if G.shape[1] != n or tuple(R.shape) != (nseq, n):
        raise ValueError("G must be n x n and R nseq x n")
    if mask_bits.dtype not in (torch.int32, torch.uint32):
        raise TypeError("mask_bits must be int32 or uint32 words")
    _dev(mask_bits, "mask_bits", mask_bits.dtype, 2)
    if tuple(mask_bits.shape) != (nseq, (n + 31) // 32):
        raise ValueError("mask_bits disagree with G and last_pick")
    dev = G.device
    idx_out = _out(idx_out, "idx_out", torch.int32, nseq, dev)
    score_out = _out(score_out, "score_out", torch.float32, nseq, dev, want_score)
    with _on(dev):
        rc = L.vs_diversity_step_gram_sum(_ptr(G), n, G.stride(0), _ptr(last_pick), _ptr(R),
                                          R.stride(0), _ptr(mask_bits), nseq, _ptr(idx_out),
                                          _ptr(score_out), _stream(dev))
    _check(rc, "vs_diversity_step_gram_sum")
    return idx_out, score_out


def _map_shape(nc, map_shape):
    rows, cols = (int(v) for v in map_shape)
    if rows * cols != nc:
        raise ValueError(f"map {rows}x{cols} does not hold {nc} neurons")
    return rows, cols


def _csr_args(indptr, indices, values):
    torch = _torch()
    _dev(indptr, "indptr", torch.int32, 1)
    _dev(indices, "indices", torch.int32, 1)
    _dev(values, "values", torch.float32, 1)
    n = indptr.numel() - 1
    nnz = indices.numel()
    if values.numel() != nnz:
        raise ValueError("indices and values differ in length")
    return n, nnz


def vs_som_update(X, bmu, C, map_shape, sigma: float, radius: int, workspace=None):
    """Batch SOM update of the neuron-major codebook C (rows*cols x d) in
    place from the dense rows X and their BMU indices (see include/vs.h)."""
    torch = _torch()
    L = lib()
    _dev(X, "X", torch.float32, 2)
    _dev(bmu, "bmu", torch.int32, 1)
    _dev(C, "C", torch.float32, 2)
    n, d = X.shape
    nc = C.shape[0]
    if C.shape[1] != d or bmu.numel() != n:
        raise ValueError("X, bmu and C disagree in shape")
    rows, cols = _map_shape(nc, map_shape)
    dev = C.device
    ws = _workspace(L.vs_som_update_workspace(rows, cols, d), dev, workspace)
    with _on(dev):
        rc = L.vs_som_update(_ptr(X), n, d, _ptr(bmu), _ptr(C), rows, cols, float(sigma),
                             int(radius), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_som_update")
    return C


def vs_som_update_csr(indptr, indices, values, bmu, CB, map_shape, d: int, sigma: float,
                      radius: int, workspace=None):
    """Batch SOM update, CSR rows, of the 64-neuron blocked codebook CB (the
    layout vs_csr_block_codebook writes) in place."""
    torch = _torch()
    L = lib()
    n, nnz = _csr_args(indptr, indices, values)
    _dev(bmu, "bmu", torch.int32, 1)
    _dev(CB, "CB", torch.float32, 1)
    rows, cols = (int(v) for v in map_shape)
    nc = rows * cols
    if bmu.numel() != n:
        raise ValueError("bmu must hold one index per row")
    if CB.numel() < ((nc + 63) // 64) * 64 * d:
        raise ValueError("CB is smaller than the blocked layout of rows*cols x d")
    dev = CB.device
    ws = _workspace(L.vs_som_update_workspace(rows, cols, d), dev, workspace)
    with _on(dev):
        rc = L.vs_som_update_csr(_ptr(indptr), _ptr(indices) if nnz else None,
                                 _ptr(values) if nnz else None, n, nnz, _ptr(bmu), _ptr(CB),
                                 rows, cols, d, float(sigma), int(radius), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_som_update_csr")
    return CB


def vs_som_qe(score, qe_out=None):
    """Quantisation error (float64 tensor of one element) from BMU scores."""
    torch = _torch()
    L = lib()
    _dev(score, "score", torch.float32, 1)
    dev = score.device
    qe_out = _out(qe_out, "qe_out", torch.float64, 1, dev)
    with _on(dev):
        rc = L.vs_som_qe(_ptr(score), score.numel(), _ptr(qe_out), _stream(dev))
    _check(rc, "vs_som_qe")
    return qe_out


def vs_som_epoch(X, C, map_shape, sigma: float, radius: int, bmu_out=None, score_out=None,
                 qe_out=None, workspace=None):
    """One SOM epoch on dense rows: BMU search, quantisation error, batch
    update of C in place.  Returns (bmu, score, qe)."""
    torch = _torch()
    L = lib()
    _dev(X, "X", torch.float32, 2)
    _dev(C, "C", torch.float32, 2)
    n, d = X.shape
    nc = C.shape[0]
    if C.shape[1] != d:
        raise ValueError("X and C must have the same number of columns")
    rows, cols = _map_shape(nc, map_shape)
    dev = C.device
    bmu_out = _out(bmu_out, "bmu_out", torch.int32, n, dev)
    score_out = _out(score_out, "score_out", torch.float32, n, dev)
    qe_out = _out(qe_out, "qe_out", torch.float64, 1, dev)
    ws = _workspace(L.vs_som_epoch_workspace(n, rows, cols, d), dev, workspace)
    with _on(dev):
        rc = L.vs_som_epoch(_ptr(X), n, d, _ptr(C), rows, cols, float(sigma), int(radius),
                            _ptr(bmu_out), _ptr(score_out), _ptr(qe_out), _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_som_epoch")
    return bmu_out, score_out, qe_out


def vs_som_epoch_csr(indptr, indices, values, CB, map_shape, d: int, sigma: float, radius: int,
                     bmu_out=None, score_out=None, qe_out=None, workspace=None):
    """One SOM epoch on CSR rows over the blocked codebook CB: BMU search,
    quantisation error, batch update of CB in place.  Returns (bmu, score, qe)."""
    torch = _torch()
    L = lib()
    n, nnz = _csr_args(indptr, indices, values)
    _dev(CB, "CB", torch.float32, 1)
    rows, cols = (int(v) for v in map_shape)
    nc = rows * cols
    if CB.numel() < ((nc + 63) // 64) * 64 * d:
        raise ValueError("CB is smaller than the blocked layout of rows*cols x d")
    dev = CB.device
    bmu_out = _out(bmu_out, "bmu_out", torch.int32, n, dev)
    score_out = _out(score_out, "score_out", torch.float32, n, dev)
    qe_out = _out(qe_out, "qe_out", torch.float64, 1, dev)
    ws = _workspace(L.vs_som_epoch_csr_workspace(n, rows, cols, d), dev, workspace)
    with _on(dev):
        rc = L.vs_som_epoch_csr(_ptr(indptr), _ptr(indices) if nnz else None,
                                _ptr(values) if nnz else None, n, nnz, _ptr(CB), rows, cols, d,
                                float(sigma), int(radius), _ptr(bmu_out), _ptr(score_out),
                                _ptr(qe_out), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(dev))
    _check(rc, "vs_som_epoch_csr")
    return bmu_out, score_out, qe_out


def vs_csr_blocked_to_f16(CB, nc: int, d: int, out=None):
    """The fp16 128-neuron blocked copy of a 64-neuron blocked fp32 codebook."""
    torch = _torch()
    L = lib()
    _dev(CB, "CB", torch.float32, 1)
    if CB.numel() < ((nc + 63) // 64) * 64 * d:
        raise ValueError("CB is smaller than the blocked layout of nc x d")
    out = _out(out, "out", torch.float16, L.vs_csr_blocked_f16_bytes(nc, d) // 2, CB.device)
    with _on(CB.device):
        rc = L.vs_csr_blocked_to_f16(_ptr(CB), nc, d, _ptr(out), _stream(CB.device))
    _check(rc, "vs_csr_blocked_to_f16")
    return out


def vs_som_epoch_csr_f16(indptr, indices, values, CB, map_shape, d: int, sigma: float,
                         radius: int, CB16=None, bmu_out=None, score_out=None, qe_out=None,
                         workspace=None):
    """One SOM epoch on CSR rows searching an fp16 copy (CB16) of the fp32
    blocked codebook CB, updating CB in place.  Returns (bmu, score, qe)."""
    torch = _torch()
    L = lib()
    n, nnz = _csr_args(indptr, indices, values)
    _dev(CB, "CB", torch.float32, 1)
    rows, cols = (int(v) for v in map_shape)
    nc = rows * cols
    if CB.numel() < ((nc + 63) // 64) * 64 * d:
        raise ValueError("CB is smaller than the blocked layout of rows*cols x d")
    dev = CB.device
    CB16 = _out(CB16, "CB16", torch.float16, L.vs_csr_blocked_f16_bytes(nc, d) // 2, dev)
    bmu_out = _out(bmu_out, "bmu_out", torch.int32, n, dev)
    score_out = _out(score_out, "score_out", torch.float32, n, dev)
    qe_out = _out(qe_out, "qe_out", torch.float64, 1, dev)
    ws = _workspace(L.vs_som_epoch_csr_workspace(n, rows, cols, d), dev, workspace)
    with _on(dev):
        rc = L.vs_som_epoch_csr_f16(_ptr(indptr), _ptr(indices) if nnz else None,
                                    _ptr(values) if nnz else None, n, nnz, _ptr(CB), _ptr(CB16),
                                    rows, cols, d, float(sigma), int(radius), _ptr(bmu_out),
                                    _ptr(score_out), _ptr(qe_out), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "vs_som_epoch_csr_f16")
    return bmu_out, score_out, qe_out


def vs_candidate_norms(C, feature_major: bool = False, out=None):
    """Squared L2 norms (float32) of the rows of C, or of its columns."""
    torch = _torch()
    L = lib()
    _dev(C, "C", torch.float32, 2)
    if feature_major:
        d, nc = C.shape
    else:
        nc, d = C.shape
    out = _out(out, "out", torch.float32, nc, C.device)
    with _on(C.device):
        rc = L.vs_candidate_norms(_ptr(C), nc, d, int(bool(feature_major)), _ptr(out),
                                  _stream(C.device))
    _check(rc, "vs_candidate_norms")
    return out


def vs_tile_rows(cache_bytes: int, d: int, bytes_per_value: int = 4) -> int:
    return int(lib().vs_tile_rows(cache_bytes, d, bytes_per_value))


def mask_words(n: int) -> int:
    return (n + 31) // 32


class KernelTimer:
    """Sum of the dominant kernel's durations (HIP events on the call's stream)."""

    def __init__(self, max_launches: int = 4096):
        self.max = max_launches
        self.ms = None
        self.launches = None

    def __enter__(self):
        _check(lib().vs_timing_enable(self.max), "vs_timing_enable")
        return self

    def __exit__(self, *exc):
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        _check(lib().vs_timing_read(ctypes.byref(ms), ctypes.byref(n)), "vs_timing_read")
        self.ms, self.launches = ms.value, n.value
        self.name = lib().vs_timing_kernel_name().decode()
        return False
