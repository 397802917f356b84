"""CPU oracle for token-block MXFP8 causal packed attention (the FLAMIA method).

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()`` and by
the CPU-baseline leg of ``bench.py``.  The product path (the HIP library and its Python
binding) never imports, links or runs anything in this directory, and the two share no
code.  The arithmetic lives in ``flamia_oracle.c`` (plain C, double precision); this
module only marshals numpy arrays through ctypes.

Tensor conventions: BF16 tensors are passed as numpy ``uint16`` bit patterns with layout
[T, H, d]; codes are ``uint8`` [T, H, d]; scale tables ``uint8`` [H, T] holding the E8M0
byte (exponent + 127); LSE and D are ``float32`` [H, T]; ``cu`` is int32 [n_docs + 1].
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "flamia_oracle.c")
_SO = os.path.join(_HERE, "_build", "liboracle.so")
_lib = None


def build():
    """Compile the oracle with gcc (-O2, no fast-math, no FP contraction, OpenMP)."""
    os.makedirs(os.path.dirname(_SO), exist_ok=True)
    tmp = _SO + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-shared",
                           "-fPIC", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_SO)
        _lib.orc_e4m3_decode.restype = ctypes.c_double
        _lib.orc_e4m3_rne.restype = ctypes.c_uint8
        _lib.orc_e8m0_roundup.restype = ctypes.c_int
        _lib.orc_e8m0_floor.restype = ctypes.c_int
        _lib.orc_e2m1_decode.restype = ctypes.c_double
        _lib.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        _lib.orc_e2m1_rne.restype = ctypes.c_uint8
        _lib.orc_e8m0_roundup4.restype = ctypes.c_int
        for f in ("orc_e4m3_rne", "orc_e8m0_roundup", "orc_e8m0_floor", "orc_e2m1_rne", "orc_e8m0_roundup4"):
            getattr(_lib, f).argtypes = [ctypes.c_double]
        _lib.orc_worklist.restype = ctypes.c_int
        _lib.orc_schedule_dynamic.restype = ctypes.c_int
        _lib.orc_small_docs.restype = ctypes.c_int
        _lib.orc_num_threads.restype = ctypes.c_int
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads():
    return lib().orc_num_threads()


# ---------------------------------------------------------------------------------------
# number formats
def e4m3_rne(y):
    y = _c(y, np.float64)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e4m3_rne_array(_p(y), _p(out), ctypes.c_long(y.size))
    return out


def e4m3_decode(c):
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_e4m3_decode_array(_p(c), _p(out), ctypes.c_long(c.size))
    return out


def bf16_rne(y):
    y = _c(y, np.float64)
    out = np.empty(y.shape, np.uint16)
    lib().orc_bf16_rne_array(_p(y), _p(out), ctypes.c_long(y.size))
    return out


def f16_rne(y):
    y = _c(y, np.float64)
    out = np.empty(y.shape, np.uint16)
    lib().orc_f16_rne_array(_p(y), _p(out), ctypes.c_long(y.size))
    return out


def e8m0_roundup(a):
    a = _c(a, np.float64)
    out = np.empty(a.shape, np.int32)
    lib().orc_e8m0_roundup_array(_p(a), _p(out), ctypes.c_long(a.size))
    return out


def e8m0_floor(a):
    return int(lib().orc_e8m0_floor(float(a)))


# ---------------------------------------------------------------------------------------
# the method
def quantize(x_bits, cu, floor_rule=False, hadamard=False, per_token=False):
    """Token-block quantiser: returns (codes [T,H,d] u8, scales [H,T] u8).  hadamard=True rotates
    each (token, head) row first (see hadamard()); per_token=True gives every token its own
    exponent (blocks of one token)."""
    x = _c(x_bits, np.uint16)
    T, H, d = x.shape
    cu = _c(cu, np.int32)
    codes = np.empty((T, H, d), np.uint8)
    scales = np.empty((H, T), np.uint8)
    if per_token:
        assert not floor_rule and not hadamard
        lib().orc_quantize_per_token(_p(x), T, H, d, _p(cu), len(cu) - 1, _p(codes), _p(scales))
    elif hadamard:
        assert not floor_rule
        lib().orc_quantize_hadamard(_p(x), T, H, d, _p(cu), len(cu) - 1, _p(codes), _p(scales))
    else:
        lib().orc_quantize(_p(x), T, H, d, _p(cu), len(cu) - 1, _p(codes), _p(scales), int(bool(floor_rule)))
    return codes, scales


def e2m1_decode(c):
    """Values of E2M1 codes (low nibble of each byte)."""
    c = np.asarray(c, np.uint8)
    return np.vectorize(lambda x: lib().orc_e2m1_decode(int(x) & 15), otypes=[np.float64])(c) if c.size else \
        np.zeros(c.shape)


def e2m1_rne(y):
    """Nearest E2M1 codes (ties to even, signed zero kept, beyond 6 saturated)."""
    y = np.asarray(y, np.float64)
    return np.vectorize(lambda x: lib().orc_e2m1_rne(float(x)), otypes=[np.uint8])(y) if y.size else \
        np.zeros(y.shape, np.uint8)


def e8m0_roundup4(a):
    """Smallest s with a <= 6 2^s (clamped to [-127, 127]; 0 gives -127)."""
    return int(lib().orc_e8m0_roundup4(float(a)))


def quantize_mx4(x_bits, cu, hadamard=False):
    """The 4-bit copy (E2M1 codes, one E8M0 exponent per 32 channels of a token): returns
    (codes [T,H,d/2] u8, even channel in the low nibble; scales [H,T,d/32] u8)."""
    x = _c(x_bits, np.uint16)
    T, H, d = x.shape
    cu = _c(cu, np.int32)
    codes = np.empty((T, H, d // 2), np.uint8)
    scales = np.empty((H, T, d // 32), np.uint8)
    lib().orc_quantize_mx4(_p(x), T, H, d, _p(cu), len(cu) - 1, int(bool(hadamard)), _p(codes), _p(scales))
    return codes, scales


def hadamard(x):
    """Rows of the last axis (FP32) times H / sqrt(d): FP32 butterflies, strides 1, 2, ..., d/2,
    then the FP32 multiply by RN32(1 / sqrt(d)).  Returns a new float32 array."""
    x = np.array(x, dtype=np.float32, order="C", copy=True)
    d = x.shape[-1]
    lib().orc_hadamard(_p(x), ctypes.c_long(x.size // d), d)
    return x


def unrotate_bf16(bits):
    """BF16 gradient rows (last axis d) back to the inputs' basis: BF16(hadamard(row))."""
    b = _c(bits, np.uint16)
    d = b.shape[-1]
    out = np.empty(b.shape, np.uint16)
    lib().orc_unrotate_bf16(_p(b), _p(out), ctypes.c_long(b.size // d), d)
    return out


def worklist(cu, kind, n_workers):
    """Sorted work list: int32 [n_items, 4] rows {doc, blk, cost, worker}; kind 0 = fwd, 1 = bwd,
    2 = non-causal fwd, 3 = non-causal bwd (every item of a document costs its key-tile count)."""
    cu = _c(cu, np.int32)
    n_docs = len(cu) - 1
    cap = int(sum((int(cu[k + 1] - cu[k]) + 127) // 128 for k in range(n_docs))) + 1
    out = np.empty((cap, 4), np.int32)
    n = lib().orc_worklist(_p(cu), n_docs, int(kind), int(n_workers), _p(out), cap)
    assert n >= 0
    return out[:n].copy()


def small_docs(cu):
    """Number of documents of 1 .. 8 tokens (their items close every list)."""
    cu = _c(cu, np.int32)
    return int(lib().orc_small_docs(_p(cu), len(cu) - 1))


def schedule_dynamic(cu, kind):
    """1 if a list of this kind over cu is taken dynamically (non-causal, longest document >= 4x
    the average), else 0."""
    cu = _c(cu, np.int32)
    return int(lib().orc_schedule_dynamic(_p(cu), len(cu) - 1, int(kind)))


class _Window(ctypes.Structure):
    _fields_ = [("row_lo", ctypes.c_int), ("row_hi", ctypes.c_int), ("key_lo", ctypes.c_int),
                ("key_hi", ctypes.c_int), ("head_lo", ctypes.c_int), ("head_hi", ctypes.c_int),
                ("fwd_s", ctypes.c_void_p), ("fwd_m", ctypes.c_void_p), ("fwd_p", ctypes.c_void_p),
                ("bwd_dp", ctypes.c_void_p), ("bwd_p", ctypes.c_void_p), ("bwd_ps", ctypes.c_void_p),
                ("bwd_ds", ctypes.c_void_p), ("bwd_dss", ctypes.c_void_p), ("fwd_ps", ctypes.c_void_p)]


def window_shape(win):
    """(heads, rows, keys) of a window dict {row_lo, row_hi, key_lo, key_hi, head_lo, head_hi}."""
    return (win["head_hi"] - win["head_lo"], win["row_hi"] - win["row_lo"], win["key_hi"] - win["key_lo"])


def _window(win, arrays):
    w = _Window(win["row_lo"], win["row_hi"], win["key_lo"], win["key_hi"], win["head_lo"], win["head_hi"])
    for name, a in arrays.items():
        setattr(w, name, a.ctypes.data if a is not None else None)
    return w


def _dump_arrays(win, names):
    shp = window_shape(win)
    out = {}
    for n in names:
        if n in ("fwd_s", "fwd_m", "bwd_dp"):
            out[n] = np.full(shp, np.nan, np.float64)
        else:
            out[n] = np.full(shp, 0xFF, np.uint8)
    return out


def _sel(mask, n):
    if mask is None:
        return None
    m = np.zeros(n, np.uint8)
    m[np.asarray(mask)] = 1
    return m


def fwd(q, sq, k, sk, v, sv, cu, softmax_scale=None, p_shift=8, exact_p=False, want_o64=False,
        docs=None, kv_heads=None, tail_rows=0, window=None, causal=True, precise=False, qk4=None):
    """causal=False: every key of the row's document is visible (key tiles from the document's
    last down to tile 0).  precise=True (with per-token operand scales): V's exponent is folded into
    the probability operand against the row's running maximum of visited V exponents.  Returns (O bits u16 [T,Hq,d], LSE f32 [Hq,T] in log2 units, O64 or None), plus (with
    ``window``, a dict of row/key/head bounds)
    a dict of the per-pair dumps fwd_s (score accumulator), fwd_m (running maximum), fwd_p
    (E4M3 codes), [heads][rows][keys], NaN / 0xFF where not visited.  ``docs`` / ``kv_heads``
    (index lists) restrict the work to those documents / KV heads, and tail_rows > 0 to the last
    tail_rows rows of each document; other rows are zero (O) or NaN (LSE).
    qk4 = (q4, sq4, k4, sk4), the 4-bit copies (quantize_mx4): 4-bit scores, and the probability
    operand quantised per 32-key group in the log domain (the window then also dumps fwd_ps, the
    group exponent byte of each code)."""
    if qk4 is not None and precise:
        raise ValueError("the 4-bit scores and the precision options are separate paths")
    q, k, v = _c(q, np.uint8), _c(k, np.uint8), _c(v, np.uint8)
    sq, sk, sv = _c(sq, np.uint8), _c(sk, np.uint8), _c(sv, np.uint8)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    cu = _c(cu, np.int32)
    o = np.zeros((T, Hq, d), np.uint16)
    lse = np.full((Hq, T), np.nan, np.float32)
    o64 = np.zeros((T, Hq, d), np.float64) if want_o64 else None
    sd, sk_ = _sel(docs, len(cu) - 1), _sel(kv_heads, Hkv)
    names = ("fwd_s", "fwd_m", "fwd_p") + (("fwd_ps",) if qk4 is not None else ())
    dumps = _dump_arrays(window, names) if window is not None else None
    w = _window(window, dumps) if window is not None else None
    q4 = [_c(a, np.uint8) for a in qk4] if qk4 is not None else None
    lib().orc_fwd(_p(q), _p(sq), _p(k), _p(sk), _p(v), _p(sv), T, Hq, Hkv, d, ctypes.c_double(softmax_scale),
                  _p(cu), len(cu) - 1, int(p_shift), int(bool(exact_p)), _p(o), _p(lse),
                  _p(o64) if o64 is not None else None, _p(sd) if sd is not None else None,
                  _p(sk_) if sk_ is not None else None, int(tail_rows), ctypes.byref(w) if w is not None else None,
                  int(bool(causal)), int(bool(precise)), *(_p(a) for a in q4) if q4 else (None,) * 4)
    return (o, lse, o64) + ((dumps,) if window is not None else ())


def quantize_do(do_bits, o_bits, cu, per_token=False):
    """dO quantiser + D: returns (codes, scales, D f32 [H,T]); per_token: one exponent per token."""
    do_bits, o_bits = _c(do_bits, np.uint16), _c(o_bits, np.uint16)
    T, H, d = do_bits.shape
    cu = _c(cu, np.int32)
    codes = np.empty((T, H, d), np.uint8)
    scales = np.empty((H, T), np.uint8)
    D = np.empty((H, T), np.float32)
    lib().orc_quantize_do_ex(_p(do_bits), _p(o_bits), T, H, d, _p(cu), len(cu) - 1, _p(codes), _p(scales), _p(D),
                             int(bool(per_token)))
    return codes, scales, D


def dq_exponents(sk, sv, sdo, cu, Hkv, d, causal_dq, per_token=False):
    """pi [Hq, T]: sequence-wide (causal_dq False), causal to the row's block end (True), or with
    per_token=True (the precision options) causal to the row itself."""
    sk, sv, sdo = _c(sk, np.uint8), _c(sv, np.uint8), _c(sdo, np.uint8)
    Hq, T = sdo.shape
    cu = _c(cu, np.int32)
    pi = np.empty((Hq, T), np.int16)
    mode = 2 if per_token else int(bool(causal_dq))
    lib().orc_dq_exponents(_p(sk), _p(sv), _p(sdo), T, Hq, Hkv, d, _p(cu), len(cu) - 1, mode, _p(pi))
    return pi


class _Dbg(ctypes.Structure):
    _fields_ = [("p_scale", ctypes.c_void_p), ("ds_scale", ctypes.c_void_p),
                ("p_code", ctypes.c_void_p), ("ds_code", ctypes.c_void_p)]


def bwd(q, sq, k, sk, v, sv, do, sdo, lse, D, cu, softmax_scale=None, causal_dq=False, exact=0,
        want64=False, debug=False, docs=None, kv_heads=None, tail_blocks=0, window=None, causal=True, precise=False,
        qk4=None):
    """Returns dict with dq, dk, dv (u16 BF16 bits), pi (i16 [Hq,T]) and optionally the
    double-precision values (dq64, dk64, dv64) and, for single-document calls, the block
    exponents/codes of the P and dS operands (p_scale, ds_scale [Hq,nb,nb]; p_code,
    ds_code [Hq,L,L]).  tail_blocks > 0 restricts the work to the last tail_blocks 32-query
    blocks of each document: only those rows' dQ and those keys' dK, dV are complete.  With
    ``window`` (row/key/head bounds), out["dumps"] holds the per-pair bwd_dp (D - dP), bwd_p,
    bwd_ps (Phat code, block exponent byte), bwd_ds, bwd_dss (dShat), [heads][rows][keys].
    causal=False: every key of the row's document is visible (default dQ prescale only).
    qk4 = (q4, sq4, k4, sk4): the recomputed scores take these 4-bit copies (the forward's)."""
    if qk4 is not None and precise:
        raise ValueError("the 4-bit scores and the precision options are separate paths")
    if not causal and causal_dq:
        raise ValueError("the causal dQ prescale applies to causal attention")
    if precise and not causal:
        raise ValueError("the precision options apply to causal attention")
    q, k, v, do = (_c(a, np.uint8) for a in (q, k, v, do))
    sq, sk, sv, sdo = (_c(a, np.uint8) for a in (sq, sk, sv, sdo))
    lse, D = _c(lse, np.float32), _c(D, np.float32)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    cu = _c(cu, np.int32)
    out = dict(dq=np.empty((T, Hq, d), np.uint16), dk=np.empty((T, Hkv, d), np.uint16),
               dv=np.empty((T, Hkv, d), np.uint16), pi=np.empty((Hq, T), np.int16))
    if want64:
        out.update(dq64=np.empty((T, Hq, d)), dk64=np.empty((T, Hkv, d)), dv64=np.empty((T, Hkv, d)))
    sd, sk_ = _sel(docs, len(cu) - 1), _sel(kv_heads, Hkv)
    dbg = None
    if debug:
        assert len(cu) == 2 and cu[0] == 0
        L = int(cu[1])
        nb = (L + 31) // 32
        out.update(p_scale=np.zeros((Hq, nb, nb), np.uint8), ds_scale=np.zeros((Hq, nb, nb), np.uint8),
                   p_code=np.zeros((Hq, L, L), np.uint8), ds_code=np.zeros((Hq, L, L), np.uint8))
        dbg = _Dbg(out["p_scale"].ctypes.data, out["ds_scale"].ctypes.data,
                   out["p_code"].ctypes.data, out["ds_code"].ctypes.data)
    dumps = _dump_arrays(window, ("bwd_dp", "bwd_p", "bwd_ps", "bwd_ds", "bwd_dss")) if window is not None else None
    w = _window(window, dumps) if window is not None else None
    if dumps is not None:
        out["dumps"] = dumps
    lib().orc_bwd(_p(q), _p(sq), _p(k), _p(sk), _p(v), _p(sv), _p(do), _p(sdo), _p(lse), _p(D),
                  T, Hq, Hkv, d, ctypes.c_double(softmax_scale), _p(cu), len(cu) - 1, int(bool(causal_dq)),
                  int(exact), _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["pi"]),
                  _p(out["dq64"]) if want64 else None, _p(out["dk64"]) if want64 else None,
                  _p(out["dv64"]) if want64 else None, ctypes.byref(dbg) if dbg is not None else None,
                  _p(sd) if sd is not None else None, _p(sk_) if sk_ is not None else None,
                  int(tail_blocks), ctypes.byref(w) if w is not None else None, int(bool(causal)),
                  int(bool(precise)), *((_p(_c(a, np.uint8)) for a in qk4) if qk4 is not None else (None,) * 4))
    return out


def fwd_replay(v, sv, cu, window, S, M, P, Hq, c_scale, p_shift=8, causal=True, precise=False, PS=None):
    """Forward products from given per-pair decisions (score accumulator S, running maximum M,
    codes P, [heads][rows][keys] over ``window``; PS, the 4-bit path's per-pair group exponent
    bytes, else the fixed shift).  Returns (O64 [heads][rows][d], LSE64 [heads][rows]), NaN for
    rows not replayed.  c_scale = softmax_scale * log2(e) as used."""
    v, sv = _c(v, np.uint8), _c(sv, np.uint8)
    T, Hkv, d = v.shape
    cu = _c(cu, np.int32)
    S, M, P = _c(S, np.float64), _c(M, np.float64), _c(P, np.uint8)
    nh, nr, nk = window_shape(window)
    assert S.shape == M.shape == P.shape == (nh, nr, nk)
    o64 = np.empty((nh, nr, d))
    lse64 = np.empty((nh, nr))
    w = _window(window, {})
    lib().orc_fwd_replay(_p(v), _p(sv), T, int(Hq), Hkv, d, ctypes.c_double(c_scale), _p(cu), len(cu) - 1,
                         int(p_shift), ctypes.byref(w), _p(S), _p(M), _p(P), _p(o64), _p(lse64), int(bool(causal)),
                         int(bool(precise)), _p(_c(PS, np.uint8)) if PS is not None else None)
    return o64, lse64


def bwd_replay(q, sq, k, sk, do, sdo, cu, pi, window, P, PS, DS, DSS, softmax_scale=None, causal=True):
    """Backward products from given Phat / dShat codes and block exponent bytes ([heads][rows]
    [keys] over ``window``).  Returns dict dq64 [heads][rows][d] (window heads and rows), dk64,
    dv64 [Hkv][rows][d] (keys = the window's rows), NaN where not computed."""
    q, k, do = _c(q, np.uint8), _c(k, np.uint8), _c(do, np.uint8)
    sq, sk, sdo = _c(sq, np.uint8), _c(sk, np.uint8), _c(sdo, np.uint8)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    cu = _c(cu, np.int32)
    pi = _c(pi, np.int16)
    P, PS, DS, DSS = (_c(a, np.uint8) for a in (P, PS, DS, DSS))
    nh, nr, nk = window_shape(window)
    assert P.shape == PS.shape == DS.shape == DSS.shape == (nh, nr, nk)
    out = dict(dq64=np.empty((nh, nr, d)), dk64=np.empty((Hkv, nr, d)), dv64=np.empty((Hkv, nr, d)))
    w = _window(window, {})
    lib().orc_bwd_replay(_p(q), _p(sq), _p(k), _p(sk), _p(do), _p(sdo), T, Hq, Hkv, d,
                         ctypes.c_double(softmax_scale), _p(cu), len(cu) - 1, _p(pi), ctypes.byref(w), _p(P), _p(PS),
                         _p(DS), _p(DSS), _p(out["dq64"]), _p(out["dk64"]), _p(out["dv64"]), int(bool(causal)))
    return out
