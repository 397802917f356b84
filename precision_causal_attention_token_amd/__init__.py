"""Token-block MXFP8 causal packed-document attention for AMD MI355X (gfx950).

Python binding of ``libflamia.so`` (C ABI in ``include/flamia.h``).  This module only
marshals arguments: it allocates outputs with torch on the current device, passes raw device
pointers and the current HIP stream, and raises on a non-OK status.  Every step of the path
(quantisation, work lists, forward, backward) runs in the library's HIP kernels; there is no
fallback, and importing this module without a built library fails loudly.
"""
import ctypes
import os

import torch

from . import workloads  # noqa: F401  (seeded synthetic inputs)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflamia.so")

FLAMIA_LIST_FWD = 0
FLAMIA_LIST_BWD = 1
FLAMIA_LIST_FWD_NC = 2
FLAMIA_LIST_BWD_NC = 3

EXPORTED_SYMBOLS = (
    "flamia_status_str", "flamia_worklist_bytes", "flamia_build_worklist", "flamia_quantize",
    "flamia_fwd", "flamia_bwd", "flamia_bwd_workspace_bytes", "flamia_bwd_workspace_bytes_for",
    "flamia_bwd_static", "flamia_num_workers",
)

# Default dShat store of a backward whose caller passes no workspace: large enough that calls up
# to the 65536-token, 16-head workloads run in a few chunks; the store never grows past what one
# chunk of any documents of the call's total length needs.
DEFAULT_STORE_BYTES = 4 << 30


class _QTensor(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("stride_t", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("H", ctypes.c_int32), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("hadamard", ctypes.c_int32), ("per_token", ctypes.c_int32),
                ("mx4_codes", ctypes.c_void_p), ("mx4_scales", ctypes.c_void_p)]


class _FwdArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("sq", ctypes.c_void_p), ("sk", ctypes.c_void_p), ("sv", ctypes.c_void_p),
                ("T", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("cu_seqlens", ctypes.c_void_p), ("n_docs", ctypes.c_int32),
                ("fwd_list", ctypes.c_void_p), ("o", ctypes.c_void_p), ("o_stride_t", ctypes.c_int64),
                ("o_stride_h", ctypes.c_int64), ("lse", ctypes.c_void_p), ("non_causal", ctypes.c_int32),
                ("precise", ctypes.c_int32), ("q4", ctypes.c_void_p), ("sq4", ctypes.c_void_p),
                ("k4", ctypes.c_void_p), ("sk4", ctypes.c_void_p)]


class _BwdArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("dO", ctypes.c_void_p),
                ("sq", ctypes.c_void_p), ("sk", ctypes.c_void_p), ("sv", ctypes.c_void_p), ("sdO", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("D", ctypes.c_void_p),
                ("T", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("cu_seqlens", ctypes.c_void_p), ("n_docs", ctypes.c_int32),
                ("fwd_list", ctypes.c_void_p), ("bwd_list", ctypes.c_void_p),
                ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
                ("dq_stride_t", ctypes.c_int64), ("dq_stride_h", ctypes.c_int64),
                ("dk_stride_t", ctypes.c_int64), ("dk_stride_h", ctypes.c_int64),
                ("dv_stride_t", ctypes.c_int64), ("dv_stride_h", ctypes.c_int64),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("causal_dq_scale", ctypes.c_int32), ("dq_exp_out", ctypes.c_void_p),
                ("non_causal", ctypes.c_int32), ("hadamard", ctypes.c_int32), ("precise", ctypes.c_int32),
                ("q4", ctypes.c_void_p), ("sq4", ctypes.c_void_p), ("k4", ctypes.c_void_p), ("sk4", ctypes.c_void_p),
                ("max_doc_len", ctypes.c_int32)]


_lib = None


def load_library(path=LIB_PATH):
    """Load libflamia.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libflamia.so is not built (%s); run `python -m "
                           "precision_causal_attention_token_amd.build`" % path)
    lib = ctypes.CDLL(path)
    lib.flamia_status_str.restype = ctypes.c_char_p
    lib.flamia_status_str.argtypes = [ctypes.c_int]
    lib.flamia_worklist_bytes.restype = ctypes.c_size_t
    lib.flamia_worklist_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.flamia_build_worklist.restype = ctypes.c_int
    lib.flamia_build_worklist.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.flamia_quantize.restype = ctypes.c_int
    lib.flamia_quantize.argtypes = [ctypes.POINTER(_QTensor), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.flamia_fwd.restype = ctypes.c_int
    lib.flamia_fwd.argtypes = [ctypes.POINTER(_FwdArgs), ctypes.c_void_p]
    lib.flamia_bwd.restype = ctypes.c_int
    lib.flamia_bwd.argtypes = [ctypes.POINTER(_BwdArgs), ctypes.c_void_p]
    lib.flamia_bwd_static.restype = ctypes.c_int
    lib.flamia_bwd_static.argtypes = [ctypes.POINTER(_BwdArgs), ctypes.c_void_p]
    lib.flamia_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.flamia_bwd_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_size_t]
    lib.flamia_bwd_workspace_bytes_for.restype = ctypes.c_size_t
    lib.flamia_bwd_workspace_bytes_for.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_int32, ctypes.c_int32]
    lib.flamia_num_workers.restype = ctypes.c_int32
    lib.flamia_num_workers.argtypes = []
    _lib = lib
    return lib


class FlamiaError(RuntimeError):
    pass


def _check(status):
    if status != 0:
        raise FlamiaError("libflamia: %s (status %d)" % (load_library().flamia_status_str(status).decode(), status))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check_bf16(x, name):
    if not x.is_cuda or x.dtype != torch.bfloat16 or x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("%s must be a CUDA bf16 tensor [T, H, d] with a contiguous last dim" % name)


def _check_cu(cu):
    if not cu.is_cuda or cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous CUDA int32 vector")
    return cu.numel() - 1


def num_workers():
    return int(load_library().flamia_num_workers())


# ----------------------------------------------------------------------------------------
def build_worklist(cu_seqlens, T, kind, n_workers=None):
    """Sorted work list (int32 buffer: header {n_items, kind, n_docs, counters} + 4 ints per item,
    then the forward's unit counters; `counters` is their word position for a list marked
    dynamic, else 0)."""
    lib = load_library()
    n_docs = _check_cu(cu_seqlens)
    nbytes = lib.flamia_worklist_bytes(n_docs, int(T), int(kind))
    buf = torch.empty((nbytes + 3) // 4, dtype=torch.int32, device=cu_seqlens.device)
    if n_workers is None:
        n_workers = num_workers()
    _check(lib.flamia_build_worklist(_ptr(cu_seqlens), n_docs, int(T), int(kind), int(n_workers), _ptr(buf),
                                     buf.numel() * 4, _stream()))
    return buf


def worklist_items(buf):
    """Host view of a list buffer: (n_items, int32 tensor [n_items, 4]) (synchronises)."""
    n = int(buf[0].item())
    return n, buf[4:4 + 4 * n].view(n, 4)


def quantize(xs, cu_seqlens, hadamard=False, per_token=False, mx4=False):
    """Token-block MXFP8 quantisation of up to three BF16 tensors [T, H, d] in one launch.
    hadamard: a bool for every tensor or one per tensor (rows rotated by H / sqrt(d) first; Q
    and K of a training call); per_token: one exponent per token (the precision options);
    mx4: a bool for every tensor or one per tensor, also write the 4-bit copy for the scores.
    Returns a list of (codes u8 [T, H, d], scales u8 [H, T]), with mx4 followed by the 4-bit
    copy (codes u8 [T, H, d/2], scales u8 [H, T, d/32]) in each tensor's tuple."""
    lib = load_library()
    n_docs = _check_cu(cu_seqlens)
    T, _, d = xs[0].shape
    arr = (_QTensor * len(xs))()
    outs = []
    rot = [bool(hadamard)] * len(xs) if isinstance(hadamard, bool) else [bool(r) for r in hadamard]
    if len(rot) != len(xs):
        raise ValueError("one hadamard flag per tensor")
    four = [bool(mx4)] * len(xs) if isinstance(mx4, bool) else [bool(r) for r in mx4]
    if len(four) != len(xs):
        raise ValueError("one mx4 flag per tensor")
    for i, x in enumerate(xs):
        _check_bf16(x, "x")
        if x.shape[0] != T or x.shape[2] != d:
            raise ValueError("tensors must share T and d")
        H = x.shape[1]
        codes = torch.empty((T, H, d), dtype=torch.uint8, device=x.device)
        scales = torch.empty((H, T), dtype=torch.uint8, device=x.device)
        c4 = s4 = None
        if four[i]:
            c4 = torch.empty((T, H, d // 2), dtype=torch.uint8, device=x.device)
            s4 = torch.empty((H, T, d // 32), dtype=torch.uint8, device=x.device)
        arr[i] = _QTensor(x.data_ptr(), x.stride(0), x.stride(1), H, codes.data_ptr(), scales.data_ptr(), int(rot[i]),
                          int(bool(per_token)), c4.data_ptr() if four[i] else None,
                          s4.data_ptr() if four[i] else None)
        outs.append((codes, scales, c4, s4) if four[i] else (codes, scales))
    _check(lib.flamia_quantize(arr, len(xs), T, d, _ptr(cu_seqlens), n_docs, None, 0, 0, None, _stream()))
    return outs


def quantize_do(do, o, cu_seqlens, per_token=False):
    """dO quantisation plus D = deq(dO) . O (per_token: one exponent per token).  Returns (codes,
    scales, D f32 [H, T])."""
    lib = load_library()
    n_docs = _check_cu(cu_seqlens)
    _check_bf16(do, "do")
    _check_bf16(o, "o")
    T, H, d = do.shape
    codes = torch.empty((T, H, d), dtype=torch.uint8, device=do.device)
    scales = torch.empty((H, T), dtype=torch.uint8, device=do.device)
    D = torch.empty((H, T), dtype=torch.float32, device=do.device)
    arr = (_QTensor * 1)()
    arr[0] = _QTensor(do.data_ptr(), do.stride(0), do.stride(1), H, codes.data_ptr(), scales.data_ptr(), 0,
                      int(bool(per_token)))
    _check(lib.flamia_quantize(arr, 1, T, d, _ptr(cu_seqlens), n_docs, _ptr(o), o.stride(0), o.stride(1),
                               _ptr(D), _stream()))
    return codes, scales, D


def fwd(q, k, v, cu_seqlens, fwd_list, softmax_scale=None, out=None, causal=True, precise=False, qk4=False):
    """Forward on quantised operands.  q, k, v are (codes, scales) pairs; causal=False lets every
    row see every key of its document.  qk4=True: q and k are quantize(..., mx4=True) tuples and
    the scores take their 4-bit copies (log-domain probability operand).  Returns (O bf16
    [T, Hq, d], LSE f32 [Hq, T] in log2 units)."""
    lib = load_library()
    n_docs = _check_cu(cu_seqlens)
    four = (q[2].data_ptr(), q[3].data_ptr(), k[2].data_ptr(), k[3].data_ptr()) if qk4 else (None,) * 4
    (qc, qs), (kc, ks), (vc, vs) = q[:2], k[:2], v
    T, Hq, d = qc.shape
    Hkv = kc.shape[1]
    o = out if out is not None else torch.empty((T, Hq, d), dtype=torch.bfloat16, device=qc.device)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=qc.device)
    a = _FwdArgs(qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), qs.data_ptr(), ks.data_ptr(), vs.data_ptr(),
                 T, Hq, Hkv, d, float(softmax_scale or 0.0), cu_seqlens.data_ptr(), n_docs, fwd_list.data_ptr(),
                 o.data_ptr(), o.stride(0), o.stride(1), lse.data_ptr(), int(not causal), int(bool(precise)), *four)
    _check(lib.flamia_fwd(ctypes.byref(a), _stream()))
    return o, lse


def bwd_workspace_bytes(n_docs, T, Hq, d, store_budget=DEFAULT_STORE_BYTES):
    """Backward workspace bytes for n_docs documents of total length T (sizes only; a store of
    about store_budget bytes, 0 for the smallest accepted)."""
    return int(load_library().flamia_bwd_workspace_bytes(int(n_docs), int(T), int(Hq), int(d), int(store_budget)))


def bwd_workspace_bytes_for(cu_seqlens_host, T, Hq, d, causal=True):
    """Workspace with which a backward over these documents runs as one chunk (cu_seqlens_host:
    a host int32 array the caller already holds)."""
    import numpy as np
    cu = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    n_docs = cu.size - 1
    ptr = cu.ctypes.data_as(ctypes.c_void_p) if n_docs > 0 else None
    return int(load_library().flamia_bwd_workspace_bytes_for(ptr, n_docs, int(T), int(Hq), int(d),
                                                                      int(not causal)))


def bwd(q, k, v, do, lse, D, cu_seqlens, lists, softmax_scale=None, causal_dq_scale=False, want_pi=False,
        workspace=None, static_scratch=False, causal=True, hadamard=False, precise=False, qk4=False,
        max_doc_len=0):
    """Backward on quantised operands.  q, k, v, do are (codes, scales) pairs; lse, D f32 [Hq, T];
    lists: the micro-batch's Lists.  workspace: a uint8 CUDA tensor of at least
    bwd_workspace_bytes(n_docs, T, Hq, d, 0) bytes, or None to allocate one with the default
    store (DEFAULT_STORE_BYTES).
    static_scratch=True calls flamia_bwd_static instead (the library's static device scratch; no
    workspace is allocated or passed).
    hadamard=True: Q and K were quantised rotated; dq and dk are rotated back.
    qk4=True: q and k are quantize(..., mx4=True) tuples; the scores take their 4-bit copies.
    max_doc_len: a host bound of the longest document (0: none); the key-tile chunks are then
    launched for documents no longer than it (fewer empty launches).  A bound below the longest
    document can leave the call unrun: bwd_status(workspace) then reads status 3.
    Returns (dq, dk, dv) BF16, plus the prescale exponents pi int16 [Hq, T] if want_pi."""
    lib = load_library()
    n_docs = _check_cu(cu_seqlens)
    four = (q[2].data_ptr(), q[3].data_ptr(), k[2].data_ptr(), k[3].data_ptr()) if qk4 else (None,) * 4
    (qc, qs), (kc, ks), (vc, vs), (dc, dsc) = q[:2], k[:2], v, do
    T, Hq, d = qc.shape
    Hkv = kc.shape[1]
    dev = qc.device
    dq = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
    dk = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=dev)
    dv = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=dev)
    if workspace is None and not static_scratch:
        workspace = torch.empty(bwd_workspace_bytes(n_docs, T, Hq, d), dtype=torch.uint8, device=dev)
    pi = torch.empty((Hq, T), dtype=torch.int16, device=dev) if want_pi else None
    a = _BwdArgs(qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), dc.data_ptr(),
                 qs.data_ptr(), ks.data_ptr(), vs.data_ptr(), dsc.data_ptr(), lse.data_ptr(), D.data_ptr(),
                 T, Hq, Hkv, d, float(softmax_scale or 0.0), cu_seqlens.data_ptr(), n_docs,
                 lists.fwd.data_ptr(), lists.bwd.data_ptr(),
                 dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dq.stride(0), dq.stride(1), dk.stride(0), dk.stride(1),
                 dv.stride(0), dv.stride(1), workspace.data_ptr() if workspace is not None else None,
                 workspace.numel() if workspace is not None else 0, int(bool(causal_dq_scale)),
                 pi.data_ptr() if pi is not None else None, int(not causal), int(bool(hadamard)),
                 int(bool(precise)), *four, int(max_doc_len))
    _check((lib.flamia_bwd_static if static_scratch else lib.flamia_bwd)(ctypes.byref(a), _stream()))
    return (dq, dk, dv, pi) if want_pi else (dq, dk, dv)


def bwd_status(workspace):
    """Header of the last backward that used `workspace`: (status, key-tile chunks run); status
    0 once the backward has laid out its chunks (synchronises)."""
    h = workspace[:8].view(torch.int32).cpu()
    return int(h[0]), int(h[1])


class Lists:
    """Forward and backward work lists of one micro-batch (built on the GPU once, reused by every
    layer; nothing is copied to the host); causal=False builds the non-causal kinds."""

    def __init__(self, cu_seqlens, T, causal=True):
        self.fwd = build_worklist(cu_seqlens, T, FLAMIA_LIST_FWD if causal else FLAMIA_LIST_FWD_NC)
        self.bwd = build_worklist(cu_seqlens, T, FLAMIA_LIST_BWD if causal else FLAMIA_LIST_BWD_NC)


def training_call(q, k, v, do, cu_seqlens, lists=None, softmax_scale=None, causal_dq_scale=False, causal=True,
                  hadamard=False, precise=False, max_doc_len=0):
    """One attention training call: quantise Q, K, V -> forward -> quantise dO (+ D) -> backward.
    precise=True: the precision options (per-token scales in every quantiser pass, the precise
    forward and backward).  max_doc_len: as in bwd.  Returns dict with o, lse, dq, dk, dv."""
    T = q.shape[0]
    if lists is None:
        lists = Lists(cu_seqlens, T, causal)
    qz, kz, vz = quantize([q, k, v], cu_seqlens, hadamard=(hadamard, hadamard, False), per_token=precise)
    o, lse = fwd(qz, kz, vz, cu_seqlens, lists.fwd, softmax_scale, causal=causal, precise=precise)
    dc, dsc, D = quantize_do(do, o, cu_seqlens, per_token=precise)
    dq, dk, dv = bwd(qz, kz, vz, (dc, dsc), lse, D, cu_seqlens, lists, softmax_scale, causal_dq_scale,
                     causal=causal, hadamard=hadamard, precise=precise, max_doc_len=max_doc_len)
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
