"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI and check it against
the oracle on the same seeded inputs.

Acceptance bar (the benchmark spec): codes, scales, pi and work lists bit-exact; O, dQ, dK, dV cosine
>= 0.9995 and max |diff| <= 2e-2 RMS per tensor (FP64); leakage exactly 0.

How the floating-point outputs are held to the bar.  The method takes E4M3 decisions (the
probability codes of the forward, the Phat and dShat codes and their 32x32 block exponents of
the backward) on values that the GPU forms in FP32 with the FP8 matrix instruction's
accumulation and the oracle forms in FP64.  Where such a value lies within rounding of an E4M3
midpoint, either code is a correct result of the method, and one code step moves an output by
more than 2e-2 RMS in rows with few keys.  So the stage check runs the parity tests' variant of
the library (tests/_build/libflamia_debug.so, the same kernels plus copies of their per-pair
intermediates; its outputs are compared bit for bit with libflamia.so's) and checks:
  1. the forward and backward score accumulators are bit-identical, masks included;
  2. each score is the exact dot product of the codes within the FP8 instruction's accumulation
     bound, 2^-10 of the largest products of its 64-term chunks (and D - dP the same way);
  3. each running maximum is exactly the FP32 maximum the forward defines;
  4. each E4M3 decision (probability codes; Phat, dShat codes and block exponents) equals the
     oracle's rounding of the value the method defines, recomputed from the GPU's own FP32
     inputs to it, except where that value lies within the exponential's precision (2^-20
     relative) of a rounding boundary: such decisions are counted and listed;
  5. O, LSE, dQ, dK, dV equal the oracle's replay of the products on those decisions
     (oracle.fwd_replay / bwd_replay) within max |diff| <= 2e-2 RMS, plus one BF16 ulp of the
     reference (both sides round to BF16; one ulp exceeds 2e-2 RMS for elements above ~2.6 RMS),
     and the LSE within its FP32 summation bound.
The chain check then compares the whole GPU call with the oracle's own chain on the BF16
inputs at the cosine bar, and names every element beyond 2e-2 RMS + 1 ulp with the part of its
difference that the decisions account for (replay minus oracle)."""
import contextlib
import ctypes
import os
import sys

import numpy as np
import torch

import precision_causal_attention_token_amd as fl
from precision_causal_attention_token_amd import build as fl_build
from tests.helpers import bf16_bits, bits_to_f64, cosine, dequant, dequant4, rms

COS_MIN = 0.9995
MAXABS_REL = 2e-2
ACC_REL = 2.0 ** -10       # FP8 instruction accumulation bound (largest products of each 64-term chunk)
EXP_REL = 2.0 ** -20       # precision of the values E4M3 decisions are taken on (exponential, FP32 products)
LOG2E = 1.4426950408889634074


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------------------------------
# libraries
_debug_lib = None


def debug_library():
    """The parity tests' variant of the library (built by __graft_entry__.build())."""
    global _debug_lib
    if _debug_lib is None:
        if not os.path.exists(fl_build.DEBUG_LIB):
            raise RuntimeError("%s is not built; run __graft_entry__.build()" % fl_build.DEBUG_LIB)
        saved = fl._lib
        fl._lib = None
        try:
            lib = fl.load_library(fl_build.DEBUG_LIB)
        finally:
            fl._lib = saved
        lib.flamia_debug_set_dump.restype = ctypes.c_int
        _debug_lib = lib
    return _debug_lib


@contextlib.contextmanager
def using(lib):
    saved = fl._lib
    fl._lib = lib
    try:
        yield
    finally:
        fl._lib = saved


def _dump_struct(win, bufs):
    class Dump(ctypes.Structure):
        _fields_ = [(n, ctypes.c_int32) for n in ("row_lo", "row_hi", "key_lo", "key_hi", "head_lo", "head_hi")] + \
                   [(n, ctypes.c_void_p) for n in ("fwd_s", "fwd_m", "fwd_p", "bwd_s", "bwd_dp", "bwd_p", "bwd_ps",
                                                   "bwd_ds", "bwd_dss", "dq_part")] + [("n_tiles", ctypes.c_int32)] + \
                   [(n, ctypes.c_void_p) for n in ("dq_s", "dq_dp", "dq_ds", "dq_dss", "fwd_ps")]
    d = Dump(win["row_lo"], win["row_hi"], win["key_lo"], win["key_hi"], win["head_lo"], win["head_hi"])
    for n, t in bufs.items():
        setattr(d, n, t.data_ptr())
    d.n_tiles = n_key_tiles(win)
    return d


def n_key_tiles(win):
    return -(-(win["key_hi"] - win["key_lo"]) // 128)


DUMP_F32 = ("fwd_s", "fwd_m", "bwd_s", "bwd_dp", "dq_s", "dq_dp")
DUMP_U8 = ("fwd_p", "bwd_p", "bwd_ps", "bwd_ds", "bwd_dss", "dq_ds", "dq_dss", "fwd_ps")


def gpu_call(q, k, v, do, cu, causal_dq=False, softmax_scale=None, window=None, store_budget=None, causal=True,
             static_scratch=False, hadamard=False, qk4=False, max_doc_len=0):
    """Full training call on the GPU through the C ABI; returns numpy arrays (BF16 outputs as
    bit patterns).  causal=False: non-causal attention within each document.  hadamard=True: Q
    and K quantised rotated; dQ and dK are returned in the rotated basis (the backward's own
    un-rotation is checked on its own).  With `window` (row/key/head bounds) the call runs the debug variant and the
    result also holds its per-pair dumps under "dumps" ([heads][rows][keys]).  store_budget: the
    backward's dShat store (default: the binding's default; 0: the smallest accepted, many
    chunks); the key-tile chunks run are returned under "chunks".  max_doc_len: the backward's
    bound of the longest document (0: none)."""
    dev = torch.device("cuda:0")
    cu_d = torch.as_tensor(np.asarray(cu, np.int32)).to(dev)
    T = q.shape[0]
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    lib = debug_library() if window is not None else fl.load_library()
    bufs = None
    with using(lib):
        if window is not None:
            shp = (window["head_hi"] - window["head_lo"], window["row_hi"] - window["row_lo"],
                   window["key_hi"] - window["key_lo"])
            bufs = {n: torch.full(shp, float("nan"), dtype=torch.float32, device=dev) for n in DUMP_F32}
            bufs.update({n: torch.full(shp, 0xFF, dtype=torch.uint8, device=dev) for n in DUMP_U8})
            bufs["dq_part"] = torch.full(shp[:2] + (n_key_tiles(window), q.shape[2]), float("nan"),
                                         dtype=torch.float32, device=dev)
            st = lib.flamia_debug_set_dump(ctypes.byref(_dump_struct(window, bufs)))
            assert st == 0, st
        try:
            lists = fl.Lists(cu_d, T, causal)
            qz, kz, vz = fl.quantize([qd, kd, vd], cu_d, hadamard=(hadamard, hadamard, False), mx4=(qk4, qk4, False))
            o, lse = fl.fwd(qz, kz, vz, cu_d, lists.fwd, softmax_scale, causal=causal, qk4=qk4)
            dc, dsc, D = fl.quantize_do(dod, o, cu_d)
            Hq, d = q.shape[1], q.shape[2]
            budget = fl.DEFAULT_STORE_BYTES if store_budget is None else store_budget
            ws = torch.empty(fl.bwd_workspace_bytes(len(cu) - 1, T, Hq, d, budget), dtype=torch.uint8, device=dev)
            ws.fill_(0xA5)  # the workspace may hold anything on entry
            if static_scratch:
                dq, dk, dv, pi = fl.bwd(qz, kz, vz, (dc, dsc), lse, D, cu_d, lists, softmax_scale, causal_dq,
                                        want_pi=True, static_scratch=True, causal=causal, qk4=qk4)
                torch.cuda.synchronize()
                status, chunks = 0, None
            else:
                dq, dk, dv, pi = fl.bwd(qz, kz, vz, (dc, dsc), lse, D, cu_d, lists, softmax_scale, causal_dq,
                                        want_pi=True, workspace=ws, causal=causal, qk4=qk4, max_doc_len=max_doc_len)
                torch.cuda.synchronize()
                status, chunks = fl.bwd_status(ws)
            assert status == 0, 'backward workspace status'
        finally:
            if window is not None:
                lib.flamia_debug_set_dump(None)
    b = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
    n = lambda t: t.cpu().numpy()
    out = dict(q=n(qz[0]), sq=n(qz[1]), k=n(kz[0]), sk=n(kz[1]), v=n(vz[0]), sv=n(vz[1]),
               do=n(dc), sdo=n(dsc), D=n(D), o=b(o), lse=n(lse), dq=b(dq), dk=b(dk), dv=b(dv), pi=n(pi),
               chunks=chunks, causal=bool(causal), hadamard=bool(hadamard), qk4=bool(qk4))
    if qk4:
        out.update(q4=n(qz[2]), sq4=n(qz[3]), k4=n(kz[2]), sk4=n(kz[3]))
    if bufs is not None:
        out["dumps"] = {k_: n(t) for k_, t in bufs.items()}
        out["window"] = dict(window)
    return out


def same_outputs(a, b):
    """The debug variant computes exactly what the product library computes."""
    for nm in ("q", "sq", "k", "sk", "v", "sv", "do", "sdo", "D", "o", "lse", "dq", "dk", "dv", "pi") + \
            (("q4", "sq4", "k4", "sk4") if a.get("qk4") else ()):
        assert np.array_equal(a[nm].view(np.uint8), b[nm].view(np.uint8)), nm


def oracle_call(orc, q, k, v, do, cu, causal_dq=False, softmax_scale=None, docs=None, kv_heads=None,
                tail_rows=0, tail_blocks=0, causal=True, hadamard=False, qk4=False):
    """The oracle's own end-to-end chain on the BF16 inputs (hadamard: Q, K rotated before
    quantisation, dQ, dK rotated back)."""
    cu = np.asarray(cu, np.int32)
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        c, s = orc.quantize(bf16_bits(x), cu, hadamard=hadamard and name in ("q", "k"))
        out[name], out["s" + name] = c, s
    four = None
    if qk4:
        q4, k4 = (orc.quantize_mx4(bf16_bits(x), cu, hadamard=hadamard) for x in (q, k))
        four = (q4[0], q4[1], k4[0], k4[1])
        out.update(q4=q4[0], sq4=q4[1], k4=k4[0], sk4=k4[1])
    o, lse, _ = orc.fwd(out["q"], out["sq"], out["k"], out["sk"], out["v"], out["sv"], cu, softmax_scale,
                        docs=docs, kv_heads=kv_heads, tail_rows=tail_rows, causal=causal, qk4=four)
    dc, dsc, D = orc.quantize_do(bf16_bits(do), o, cu)
    g = orc.bwd(out["q"], out["sq"], out["k"], out["sk"], out["v"], out["sv"], dc, dsc, lse, D, cu, softmax_scale,
                causal_dq=causal_dq, docs=docs, kv_heads=kv_heads, tail_blocks=tail_blocks, causal=causal, qk4=four)
    out.update(do=dc, sdo=dsc, D=D, o=o, lse=lse, dq=g["dq"], dk=g["dk"], dv=g["dv"], pi=g["pi"])
    if hadamard:
        out["dq_rot"], out["dk_rot"] = out["dq"], out["dk"]
        out["dq"], out["dk"] = orc.unrotate_bf16(g["dq"]), orc.unrotate_bf16(g["dk"])
    return out


# ------------------------------------------------------------------------------------------
# bars
def bf16_ulp(x):
    """Spacing of BF16 numbers at |x| (subnormal spacing below 2^-126)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def bar_check(name, got_bits, ref64, orc, enforce=True):
    """max |gpu - ref| <= 2e-2 RMS(ref) + one BF16 ulp of ref, per element; cosine reported.
    ref64: the replay in FP64.  Returns the number of elements beyond 2e-2 RMS.  enforce=False
    reports only (dQ, whose FP16 sums are checked bit for bit on the GPU's own partials)."""
    g = bits_to_f64(got_bits).ravel()
    r = bits_to_f64(orc.bf16_rne(np.asarray(ref64, np.float64))).ravel()
    if not g.size:
        return 0
    scale = rms(r)
    diff = np.abs(g - r)
    bar = MAXABS_REL * scale
    beyond = diff > bar
    over = diff - (bar + bf16_ulp(r))
    say("  stage %-3s vs replay: cosine %.7f  bit-equal %.4f  max|diff|/rms %.3e  beyond 2e-2 rms: %d/%d "
        "(each within one BF16 ulp: %s)" % (name, cosine(g, r), float(np.mean(diff == 0)), diff.max() / max(scale, 1e-300),
                                            int(beyond.sum()), g.size, bool((over[beyond] <= 0).all())))
    if enforce:
        assert (over <= 0).all(), (name, float(over.max() / max(scale, 1e-300)))
    return int(beyond.sum())


# ------------------------------------------------------------------------------------------
# decision checks
def score_scale32(d, softmax_scale=None):
    """The FP32 score scale softmax_scale * log2(e) the kernels use (rounded once from double)."""
    ss = 1.0 / np.sqrt(d) if not softmax_scale else float(np.float32(softmax_scale))
    return np.float32(np.float64(ss) * LOG2E)


def fma32(a, b, c):
    """FP32 fused multiply-add: the product of two FP32 values is exact in FP64."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(np.float32)


def doc_map(cu, T):
    m = np.full(T, -1, np.int64)
    for i, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        m[a:b] = i
    return m


def visible_mask(cu, T, win, causal=True):
    """[rows, keys] of the window: the key belongs to the row's document (and, causal, is not
    after the row)."""
    dm = doc_map(cu, T)
    rows = np.arange(win["row_lo"], win["row_hi"])
    keys = np.arange(win["key_lo"], win["key_hi"])
    dr, dk = dm[rows], dm[keys]
    same = (dr[:, None] == dk[None, :]) & (dr[:, None] >= 0)
    return same & (keys[None, :] <= rows[:, None]) if causal else same


def _chunk_max(x):
    """Per-row maxima of |x| over 64-wide chunks of the last axis: [..., d / 64]."""
    a = np.abs(x)
    return a.reshape(a.shape[:-1] + (a.shape[-1] // 64, 64)).max(-1)


def check_decision(name, got, y, orc, vis, lo_ok=None):
    """E4M3 codes `got` against the oracle's rounding of `y` (the value the method defines, FP64):
    equal, or neighbours with y within EXP_REL of their midpoint.  Returns (mismatches, total)."""
    ref = orc.e4m3_rne(y)
    bad = (orc.e4m3_decode(ref) != orc.e4m3_decode(got)) & vis    # +0 and -0 codes are the same value
    n_bad = int(bad.sum())
    if n_bad:
        yv, gv, rv = y[bad], got[bad], ref[bad]
        dg, dr = orc.e4m3_decode(gv), orc.e4m3_decode(rv)
        mid = 0.5 * (dg + dr)
        neighbours = np.abs(gv.astype(np.int64) - rv.astype(np.int64)) == 1
        near = np.abs(yv - mid) <= EXP_REL * np.abs(yv) + 2.0 ** -149
        ok = neighbours & near
        if lo_ok is not None:
            ok |= lo_ok[bad]
        worst = np.argmax(np.abs(yv - mid) / np.maximum(np.abs(yv), 1e-300))
        say("    %s: %d of %d decisions differ from the oracle's rounding, all at a rounding boundary: %s "
            "(e.g. value %.9g, codes gpu 0x%02x / oracle 0x%02x)" % (name, n_bad, int(vis.sum()), bool(ok.all()),
                                                                   yv[worst], gv[worst], rv[worst]))
        assert ok.all(), name
    return n_bad, int(vis.sum())


def _blocks(a, r0, k0, fill):
    """[h, R, K] -> [h, R/32, 32, K/32, 32] (padded with fill), rows from r0, keys from k0 (both
    block-aligned within the document)."""
    h, R, K = a.shape
    Rp, Kp = -(-R // 32) * 32, -(-K // 32) * 32
    out = np.full((h, Rp, Kp), fill, a.dtype)
    out[:, :R, :K] = a
    return out.reshape(h, Rp // 32, 32, Kp // 32, 32)


def check_block_exponents(name, got_e, vals, vis, orc):
    """Per 32x32 document-aligned block (rows and keys of one document, window aligned to it):
    the exponent byte is the round-up exponent of the block's largest |value| over visible pairs,
    the same for every pair of the block, or one off with that maximum within EXP_REL of the
    boundary 448 2^s between them.  vals, got_e, vis: [h, rows, keys] of ONE document."""
    a = np.where(vis, np.abs(vals), 0.0)
    blk = _blocks(a, 0, 0, 0.0).max(axis=(2, 4))                       # [h, nbq, nbk]
    e_ref = orc.e8m0_roundup(blk) + 127
    gb = _blocks(got_e.astype(np.int64), 0, 0, -1)
    vb = _blocks(vis, 0, 0, False)
    any_vis = vb.any(axis=(2, 4))
    gmax = np.where(vb, gb, -1).max(axis=(2, 4))
    gmin = np.where(vb, gb, 999).min(axis=(2, 4))
    assert np.array_equal(gmax[any_vis], gmin[any_vis]), name + ": block exponent not constant"
    bad = any_vis & (gmax != e_ref)
    n_bad = int(bad.sum())
    if n_bad:
        lo = np.minimum(gmax[bad], e_ref[bad]) - 127
        near = (np.abs(gmax[bad] - e_ref[bad]) == 1) & (np.abs(blk[bad] - 448.0 * 2.0 ** lo) <= EXP_REL * blk[bad])
        say("    %s block exponents: %d of %d differ from the oracle's, all at a boundary: %s"
            % (name, n_bad, int(any_vis.sum()), bool(near.all())))
        assert near.all(), name
    return n_bad


def check_group_exponents(PS, S, M, c32, vis, cu, win, orc, causal=True):
    """4-bit scores: per (head, row, 128-key tile, 32-key group of the document) the exponent
    byte is the same for every visible key and equals the round-up exponent of
    2^(fma(max S over the group's visible keys, c, -m)) (the log-domain rule: the group's
    largest probability from its largest score), or one off with that value within EXP_REL of the
    boundary between them.  Returns the number at a boundary."""
    dm = doc_map(cu, max(win["row_hi"], win["key_hi"]))
    n_bad = 0
    for doc in sorted(set(dm[win["row_lo"]:win["row_hi"]]) - {-1}):
        a, b = int(cu[doc]), int(cu[doc + 1])
        r0, r1 = max(a, win["row_lo"]), min(b, win["row_hi"])
        rs, ks = slice(r0 - win["row_lo"], r1 - win["row_lo"]), slice(a - win["key_lo"], b - win["key_lo"])
        L = b - a
        ng = -(-L // 32)
        v = np.zeros(vis[rs, ks].shape[:1] + (ng * 32,), bool)
        v[:, :L] = vis[rs, ks]
        s = np.full(PS[:, rs, ks].shape[:2] + (ng * 32,), -np.inf, np.float32)
        s[..., :L] = np.where(vis[rs, ks], S[:, rs, ks], -np.inf)
        e = np.full(s.shape, -1, np.int64)
        e[..., :L] = PS[:, rs, ks]
        vg = v.reshape(v.shape[0], ng, 32)
        sg = s.reshape(s.shape[0], s.shape[1], ng, 32)
        eg = e.reshape(e.shape[0], e.shape[1], ng, 32)
        anyv = vg.any(-1)[None]
        gmax_e = np.where(vg[None], eg, -1).max(-1)
        gmin_e = np.where(vg[None], eg, 999).min(-1)
        assert np.array_equal(gmax_e[np.broadcast_to(anyv, gmax_e.shape)], gmin_e[np.broadcast_to(anyv, gmin_e.shape)]), \
            "group exponent not constant"
        gs = sg.max(-1)                                            # [h, r, ng] largest visible score
        m = np.stack([M[:, rs, ks][..., min(32 * j, L - 1)] for j in range(ng)], -1)   # the tile's running max
        with np.errstate(invalid="ignore", over="ignore"):
            pmax = np.exp2(fma32(gs, c32, (-m).astype(np.float32)).astype(np.float64))
        pmax = np.where(np.isfinite(gs), pmax, 0.0)
        e_ref = orc.e8m0_roundup(pmax) + 127
        sel = np.broadcast_to(anyv, gmax_e.shape)
        bad = sel & (gmax_e != e_ref)
        if bad.any():
            lo = np.minimum(gmax_e[bad], e_ref[bad]) - 127
            near = (np.abs(gmax_e[bad] - e_ref[bad]) == 1) & (np.abs(pmax[bad] - 448.0 * 2.0 ** lo) <= EXP_REL * pmax[bad])
            say("    group exponents: %d differ from the round-up, all at a boundary: %s" % (int(bad.sum()), bool(near.all())))
            assert near.all(), "group exponents"
            n_bad += int(bad.sum())
    return n_bad


def validate_forward(orc, g, cu, softmax_scale=None):
    """Checks 1-5 above for the forward: C1 (against the backward's dump), scores, running maxima,
    probability codes, and O / LSE against the oracle's replay on the GPU's decisions."""
    win, du = g["window"], g["dumps"]
    T, Hq, d = g["q"].shape
    Hkv = g["k"].shape[1]
    grp = Hq // Hkv
    c32 = score_scale32(d, softmax_scale)
    causal = g.get("causal", True)
    vis = visible_mask(cu, T, win, causal)
    hs = range(win["head_lo"], win["head_hi"])
    rows = slice(win["row_lo"], win["row_hi"])
    keys = slice(win["key_lo"], win["key_hi"])
    S, M, P = du["fwd_s"], du["fwd_m"], du["fwd_p"]
    # 1. forward and backward scores bit-identical, masks included (every entry either wrote)
    same = np.array_equal(S.view(np.uint32), du["bwd_s"].view(np.uint32))
    written = ~np.isnan(S)
    say("  C1 forward/backward scores: %d pairs written, bit-identical (masks included): %s"
        % (int(written.sum()), same))
    assert same
    assert (written[:, vis] if written.ndim == 3 else written).all(), "a visible pair was not visited"
    # 2. scores against the exact dot products of the codes (4-bit scores: of the 4-bit copies)
    qk4 = g.get("qk4", False)
    if qk4:
        qd, kd = dequant4(g["q4"], g["sq4"]), dequant4(g["k4"], g["sk4"])
    else:
        qd, kd = dequant(g["q"], g["sq"]), dequant(g["k"], g["sk"])
    worst = 0.0
    for x, h in enumerate(hs):
        ex = qd[rows, h] @ kd[keys, h // grp].T
        bound = ACC_REL * (_chunk_max(qd[rows, h]) @ _chunk_max(kd[keys, h // grp]).T) + 2.0 ** -22 * np.abs(ex)
        err = np.where(vis, np.abs(S[x].astype(np.float64) - ex), 0.0)
        worst = max(worst, float((err / np.where(vis, bound, 1.0)).max()))
        assert (err <= bound).all(), "score beyond the accumulation bound"
    say("  scores vs exact dot products: max error / bound %.3f" % worst)
    # 3. running maxima, recomputed in FP32 from the GPU's own scores (per document, key tiles
    # counted from its start, from the row's last visible tile down: the diagonal one, or the
    # document's last without the causal mask)
    dm = doc_map(cu, T)
    n_m = 0
    for doc in sorted(set(dm[win["row_lo"]:win["row_hi"]]) - {-1}):
        a, b = int(cu[doc]), int(cu[doc + 1])
        r0, r1 = max(a, win["row_lo"]), min(b, win["row_hi"])
        assert a >= win["key_lo"] and b <= win["key_hi"]
        L = b - a
        nkt = -(-L // 128)
        s_doc = S[:, r0 - win["row_lo"]:r1 - win["row_lo"], a - win["key_lo"]:b - win["key_lo"]]
        pad = np.full(s_doc.shape[:2] + (nkt * 128,), np.nan, np.float32)
        pad[..., :L] = s_doc
        t = pad.reshape(s_doc.shape[:2] + (nkt, 128))
        with np.errstate(invalid="ignore"):
            mx = np.where(np.isnan(t), -np.inf, t).max(-1).astype(np.float32)          # [h, r, tiles]
        diag = (np.arange(r0, r1) - a) // 128 if causal else np.full(r1 - r0, nkt - 1)
        above = np.arange(nkt)[None, :] > diag[:, None]                              # tiles not visited
        scaled = np.where(above[None], np.float32(-np.inf), (mx * c32).astype(np.float32))
        m_exp = np.maximum.accumulate(scaled[..., ::-1], axis=-1)[..., ::-1]         # from the diagonal down
        got = M[:, r0 - win["row_lo"]:r1 - win["row_lo"], a - win["key_lo"]:b - win["key_lo"]]
        want = np.repeat(m_exp, 128, axis=-1)[..., :L]
        v_doc = vis[r0 - win["row_lo"]:r1 - win["row_lo"], a - win["key_lo"]:b - win["key_lo"]]
        assert np.array_equal(got[:, v_doc].view(np.uint32), want[:, v_doc].view(np.uint32)), "running maximum"
        n_m += int(v_doc.sum()) * len(hs)
    say("  running maxima: %d pairs, all equal to the FP32 recomputation" % n_m)
    # 4. probability codes: E4M3 of 2^(fma(S, c, 8 - m)) (FP32 argument, exact exponential);
    # 4-bit scores: of 2^(fma(S, c, -m)) 2^-e with e the code's 32-key group exponent (PS), which
    # must be the round-up exponent of the group's largest such value, found from its largest S
    PS = du["fwd_ps"] if qk4 else None
    bias = (-M if qk4 else np.float32(8.0) - M).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        y = np.exp2(fma32(S, c32, bias).astype(np.float64))
    y = np.where(np.broadcast_to(vis, y.shape), y, 0.0)
    lo_ok = None
    if qk4:
        n_ge = check_group_exponents(PS, S, M, c32, vis, cu, win, orc, causal)
        say("  group exponents: %d at a boundary, the rest equal the oracle's round-up" % n_ge)
        # the hardware exponential returns +0 below FP32's normal range; the group exponent can
        # lift such a probability to E4M3 resolution, so a zero code is accepted there (the term
        # is below 2^-126 |V| against a row sum of at least 1)
        lo_ok = (y < 2.0 ** -126) & (orc.e4m3_decode(P) == 0)
        y = y * np.exp2(127.0 - PS.astype(np.float64))
        n_tiny = int((lo_ok & np.broadcast_to(vis, P.shape) & (orc.e4m3_decode(orc.e4m3_rne(y)) != 0)).sum())
        if n_tiny:
            say("  %d probability codes zero where p is below FP32's normal range (accepted)" % n_tiny)
    nbad, ntot = check_decision("probability codes", P, y, orc, np.broadcast_to(vis, P.shape), lo_ok=lo_ok)
    say("  probability codes: %d / %d at a rounding boundary, the rest equal the oracle's rounding" % (nbad, ntot))
    # 5. products: O and LSE against the replay on the GPU's decisions
    o64, lse64 = orc.fwd_replay(g["v"], g["sv"], cu, win, S.astype(np.float64), M.astype(np.float64), P, Hq,
                                float(c32), causal=causal, PS=PS)
    rmask = dm[win["row_lo"]:win["row_hi"]] >= 0
    got_o = np.transpose(g["o"][rows][:, win["head_lo"]:win["head_hi"]], (1, 0, 2))
    beyond = bar_check("O", got_o[:, rmask], o64[:, rmask], orc)
    lse_g = g["lse"][win["head_lo"]:win["head_hi"], rows][:, rmask].astype(np.float64)
    lse_r = lse64[:, rmask]
    nkeys = vis.sum(1)[rmask][None, :]
    # FP32 sum of nkeys terms, the exponential and logarithm, and the FP32 roundings of m + log2 l
    # and of the shift by 8 (absolute, at most an ulp of |LSE| + 16)
    lbound = LOG2E * (nkeys * 2.0 ** -23 + 2.0 ** -21) + 2.0 ** -22 * (np.abs(lse_r) + 16.0)
    lerr = np.abs(lse_g - lse_r)
    say("  stage LSE vs replay: max|diff| %.3e  max diff/bound %.3f" % (lerr.max(), (lerr / lbound).max()))
    assert (lerr <= lbound).all()
    return dict(o64=o64, lse64=lse64, beyond=beyond)


def validate_backward(orc, g, cu, causal_dq=False, softmax_scale=None):
    """Checks 2, 4, 5 for the backward: D - dP, Phat and dShat decisions, and dQ, dK, dV against
    the oracle's replay on the GPU's decisions (pi bit-exact against the oracle)."""
    win, du = g["window"], g["dumps"]
    T, Hq, d = g["q"].shape
    Hkv = g["k"].shape[1]
    grp = Hq // Hkv
    ss = 1.0 / np.sqrt(d) if not softmax_scale else softmax_scale
    c32 = score_scale32(d, softmax_scale)
    causal = g.get("causal", True)
    vis = visible_mask(cu, T, win, causal)
    hs = list(range(win["head_lo"], win["head_hi"]))
    rows = slice(win["row_lo"], win["row_hi"])
    keys = slice(win["key_lo"], win["key_hi"])
    pi = orc.dq_exponents(g["sk"], g["sv"], g["sdo"], cu, Hkv, d, causal_dq)
    assert np.array_equal(g["pi"], pi), "pi"
    # 2'. D - dP against D - the exact dot products of the codes
    dod, vd = dequant(g["do"], g["sdo"]), dequant(g["v"], g["sv"])
    DP = du["bwd_dp"]
    worst = 0.0
    for x, h in enumerate(hs):
        Dr = g["D"][h, rows].astype(np.float64)[:, None]
        ex = Dr - dod[rows, h] @ vd[keys, h // grp].T
        bound = ACC_REL * (_chunk_max(dod[rows, h]) @ _chunk_max(vd[keys, h // grp]).T + np.abs(Dr)) + \
            2.0 ** -22 * np.abs(ex)
        err = np.where(vis, np.abs(DP[x].astype(np.float64) - ex), 0.0)
        worst = max(worst, float((err / np.where(vis, bound, 1.0)).max()))
        assert (err <= bound).all(), "D - dP beyond the accumulation bound"
    say("  D - dP vs exact dot products: max error / bound %.3f" % worst)
    # 4'. Phat and dShat: P = 2^(fma(S, c, -LSE)), dS = -(P (D - dP)) in FP32; block exponents and codes
    S = du["bwd_s"]
    lse = np.stack([g["lse"][h, rows] for h in hs])[:, :, None]
    with np.errstate(invalid="ignore", over="ignore"):
        Pv = np.exp2(fma32(S, c32, -lse).astype(np.float64)).astype(np.float32)
        dS = -(Pv.astype(np.float64) * DP.astype(np.float64)).astype(np.float32)
    vis3 = np.broadcast_to(vis, S.shape)
    Pv = np.where(vis3, Pv, 0.0).astype(np.float64)
    dS = np.where(vis3, dS, 0.0).astype(np.float64)
    dm = doc_map(cu, T)
    counts = dict(p=[0, 0], ds=[0, 0], pe=0, dse=0)
    for doc in sorted(set(dm[win["row_lo"]:win["row_hi"]]) - {-1}):
        a, b = int(cu[doc]), int(cu[doc + 1])
        r0, r1 = max(a, win["row_lo"]), min(b, win["row_hi"])
        assert (r0 - a) % 32 == 0, "window rows must start on a block of the document"
        rs, ks = slice(r0 - win["row_lo"], r1 - win["row_lo"]), slice(a - win["key_lo"], b - win["key_lo"])
        v_doc = np.broadcast_to(vis[rs, ks], (len(hs),) + vis[rs, ks].shape)
        for nm, vals, code, ex in (("p", Pv, du["bwd_p"], du["bwd_ps"]), ("ds", dS, du["bwd_ds"], du["bwd_dss"])):
            counts["pe" if nm == "p" else "dse"] += check_block_exponents(
                "Phat" if nm == "p" else "dShat", ex[:, rs, ks], vals[:, rs, ks], v_doc, orc)
            y = vals[:, rs, ks] * np.exp2(127.0 - ex[:, rs, ks].astype(np.float64))
            y = np.where(v_doc, y, 0.0)
            nb, nt = check_decision("Phat codes" if nm == "p" else "dShat codes", code[:, rs, ks], y, orc, v_doc)
            counts[nm][0] += nb
            counts[nm][1] += nt
    say("  Phat: %d / %d codes and %d block exponents at a rounding boundary; dShat: %d / %d codes and %d "
        "block exponents; the rest equal the oracle's rounding" % (counts["p"][0], counts["p"][1], counts["pe"],
                                                                   counts["ds"][0], counts["ds"][1], counts["dse"]))
    # 5'. products against the replay on the GPU's decisions
    r = orc.bwd_replay(g["q"], g["sq"], g["k"], g["sk"], g["do"], g["sdo"], cu, pi, win, du["bwd_p"], du["bwd_ps"],
                       du["bwd_ds"], du["bwd_dss"], ss, causal=causal)
    rmask = dm[win["row_lo"]:win["row_hi"]] >= 0
    got_dq = np.transpose(g["dq"][rows][:, win["head_lo"]:win["head_hi"]], (1, 0, 2))
    dq16 = validate_dq_partials(orc, g, cu, pi, ss)
    same = np.array_equal(got_dq[:, rmask], dq16[:, rmask])
    say("  stage dQ vs the FP16 sum of the GPU's partials (ascending tiles, two roundings each): bit-identical %s"
        % same)
    if not same:
        bad = np.argwhere((got_dq != dq16) & rmask[None, :, None])
        say("    %d elements differ; first: %s" % (len(bad), bad[:6].tolist()))
        for hx, rx, cx in bad[:6]:
            row = win["row_lo"] + rx
            h = win["head_lo"] + hx
            pp = g["dumps"]["dq_part"][hx, rx, :, cx]
            say("    head %d row %d ch %d: gpu %r replay %r pi %d partials %s" % (
                h, row, cx, float(bits_to_f64(got_dq[hx, rx, cx])), float(bits_to_f64(dq16[hx, rx, cx])),
                int(pi[h, row]), np.array2string(pp[~np.isnan(pp)][:12], precision=9)))
    assert same, "dQ"
    beyond = {"dQ": bar_check("dQ", got_dq[:, rmask], r["dq64"][:, rmask], orc, enforce=False)}
    kv = [x for x in range(Hkv) if x * grp >= win["head_lo"] and (x + 1) * grp <= win["head_hi"]]
    kmask = rmask & ~np.isnan(r["dk64"][kv[0], :, 0]) if kv else rmask
    for nm, ref in (("dK", r["dk64"]), ("dV", r["dv64"])):
        got = np.transpose(g[nm.lower()][rows][:, kv], (1, 0, 2))
        beyond[nm] = bar_check(nm, got[:, kmask], ref[kv][:, kmask], orc)
    return dict(replay=r, kv=kv, kmask=kmask, beyond=beyond, dq16=dq16)


def validate_dq_partials(orc, g, cu, pi, ss, ds_name="bwd_ds", k_bare=False):
    """Each key tile's FP32 dQ partial (times 2^pi, as the GPU converts it to FP16) against the
    exact partial of the GPU's dShat codes and K: within the FP8 instruction's accumulation bound
    (2^-10 of the largest products of its two 64-key chunks, here bounded by chunk maxima of
    |dShat| and |K|).  Returns dQ as the method forms it from those partials: per row, tiles
    ascending, acc16 = f16(acc16 + f16(partial)), dQ = BF16(FP32(acc16) * FP32(2^-pi ss)), as
    BF16 bits [heads][rows][d]."""
    win, du = g["window"], g["dumps"]
    T, Hq, d = g["q"].shape
    grp = Hq // g["k"].shape[1]
    causal = g.get("causal", True)
    parts = du["dq_part"]                                                    # [h, r, tiles, d]
    # the dS operand's codes and exponents (ds_name, ds_name + "s"), and K with its scales or, with
    # k_bare (the precision options, whose dS operand carries K's exponent), its bare codes
    kd = dequant(g["k"], np.full_like(g["sk"], 127) if k_bare else g["sk"])
    dm = doc_map(cu, T)
    out = np.zeros(parts.shape[:2] + (d,), np.uint16)
    ss32 = np.float32(ss)
    worst = 0.0
    n_checked = 0
    for doc in sorted(set(dm[win["row_lo"]:win["row_hi"]]) - {-1}):
        a, b = int(cu[doc]), int(cu[doc + 1])
        r0, r1 = max(a, win["row_lo"]), min(b, win["row_hi"])
        rs = slice(r0 - win["row_lo"], r1 - win["row_lo"])
        L = b - a
        nkt = -(-L // 128)
        vis = visible_mask(cu, T, win, causal)[rs, a - win["key_lo"]:b - win["key_lo"]]
        last = (np.arange(r0, r1) - a) // 128 if causal else np.full(r1 - r0, nkt - 1)  # last key tile of each row
        for x, h in enumerate(range(win["head_lo"], win["head_hi"])):
            dsh = orc.e4m3_decode(du[ds_name][x, rs, a - win["key_lo"]:b - win["key_lo"]]) * \
                np.exp2(du[ds_name + "s"][x, rs, a - win["key_lo"]:b - win["key_lo"]].astype(np.float64) - 127)
            dsh = np.where(vis, dsh, 0.0)
            scale = np.exp2(pi[h, r0:r1].astype(np.float64))[:, None]
            acc = np.zeros((r1 - r0, d), np.float16)
            for kt in range(nkt):
                live = last >= kt
                if not live.any():
                    break
                ks = slice(128 * kt, min(L, 128 * kt + 128))
                kk = kd[a + ks.start:a + ks.stop, h // grp]
                ex = (dsh[:, ks] @ kk) * scale
                cmax_s = np.stack([np.abs(dsh[:, ks][:, c:c + 64]).max(1) for c in range(0, ks.stop - ks.start, 64)], 1)
                cmax_k = np.stack([np.abs(kk[c:c + 64]).max(0) for c in range(0, ks.stop - ks.start, 64)], 0)
                bound = ACC_REL * (cmax_s @ cmax_k) * scale + 2.0 ** -23 * np.abs(ex)
                gp = parts[x, rs, kt]
                assert not np.isnan(gp[live]).any(), "a dQ partial was not formed"
                err = np.abs(gp[live].astype(np.float64) - ex[live])
                worst = max(worst, float((err / np.maximum(bound[live], 1e-300)).max()))
                assert (err <= bound[live]).all(), "dQ partial beyond the accumulation bound"
                n_checked += int(live.sum()) * d
                acc = np.where(live[:, None], (acc + gp.astype(np.float16)).astype(np.float16), acc)
            down = (np.exp2(-pi[h, r0:r1].astype(np.float64)).astype(np.float32) * ss32).astype(np.float32)
            val = (acc.astype(np.float32) * down[:, None]).astype(np.float32)
            out[x, rs] = bf16_bits(torch.from_numpy(val).to(torch.bfloat16))
    say("  dQ partials: %d values vs the exact partials of the GPU's dShat codes, max error / bound %.3f"
        % (n_checked, worst))
    return out


def check_row_exponents(name, got_e, vals, vis, orc):
    """Per (row, 32-key block of one document): the exponent byte is the round-up exponent of the
    row's largest |value| over the block's visible keys, the same for every key of the block, or
    one off with that maximum within EXP_REL of the boundary between them.  [h, rows, keys] of ONE
    document, keys from its start."""
    h, R, K = vals.shape
    Kp = -(-K // 32) * 32
    a = np.zeros((h, R, Kp))
    a[..., :K] = np.where(vis, np.abs(vals), 0.0)
    rmax = a.reshape(h, R, Kp // 32, 32).max(-1)                         # [h, R, nbk]
    e_ref = orc.e8m0_roundup(rmax) + 127
    ge = np.full((h, R, Kp), -1, np.int64)
    ge[..., :K] = got_e
    vb = np.zeros((h, R, Kp), bool)
    vb[..., :K] = vis
    gb, vb = ge.reshape(h, R, Kp // 32, 32), vb.reshape(h, R, Kp // 32, 32)
    any_vis = vb.any(-1)
    gmax = np.where(vb, gb, -1).max(-1)
    gmin = np.where(vb, gb, 999).min(-1)
    assert np.array_equal(gmax[any_vis], gmin[any_vis]), name + ": row exponent not constant over the block"
    bad = any_vis & (gmax != e_ref)
    n_bad = int(bad.sum())
    if n_bad:
        lo = np.minimum(gmax[bad], e_ref[bad]) - 127
        near = (np.abs(gmax[bad] - e_ref[bad]) == 1) & (np.abs(rmax[bad] - 448.0 * 2.0 ** lo) <= EXP_REL * rmax[bad])
        say("    %s row exponents: %d of %d differ from the oracle's, all at a boundary: %s"
            % (name, n_bad, int(any_vis.sum()), bool(near.all())))
        assert near.all(), name
    return n_bad


def validate_backward_precise(orc, g, cu, softmax_scale=None):
    """The precision options' backward (causal, per-token scales): checks 2, 4, 5 as in
    validate_backward, on the folded operands.  Key-tile pass: D - dP as accumulated (times
    2^(e(Q_i) - e(dO_i))), P'' = P 2^e(dO_i) and dS'' = dS 2^e(Q_i) with their 32x32 block
    exponents, and dK, dV replayed from them with Q's and dO's bare codes.  dQ pass: its scores
    bit-identical to the key-tile pass's, its dP - D, dS' = dS 2^e(K_j) with one exponent per
    (row, 32-key block), its partials, and dQ replayed with K's bare codes."""
    win, du = g["window"], g["dumps"]
    T, Hq, d = g["q"].shape
    Hkv = g["k"].shape[1]
    grp = Hq // Hkv
    ss = 1.0 / np.sqrt(d) if not softmax_scale else softmax_scale
    c32 = score_scale32(d, softmax_scale)
    vis = visible_mask(cu, T, win, True)
    hs = list(range(win["head_lo"], win["head_hi"]))
    rows = slice(win["row_lo"], win["row_hi"])
    keys = slice(win["key_lo"], win["key_hi"])
    pi = orc.dq_exponents(g["sk"], g["sv"], g["sdo"], cu, Hkv, d, True, per_token=True)
    assert np.array_equal(g["pi"], pi), "pi"
    eq = np.stack([g["sq"][h, rows] for h in hs]).astype(np.float64)[:, :, None] - 127
    edo = np.stack([g["sdo"][h, rows] for h in hs]).astype(np.float64)[:, :, None] - 127
    # 2'. the key-tile pass's folded D - dP and the dQ pass's dP - D against the exact dot products
    dod, vd = dequant(g["do"], g["sdo"]), dequant(g["v"], g["sv"])
    DP, DQP = du["bwd_dp"], du["dq_dp"]
    worst = [0.0, 0.0]
    for x, h in enumerate(hs):
        Dr = g["D"][h, rows].astype(np.float64)[:, None]
        ex = Dr - dod[rows, h] @ vd[keys, h // grp].T
        bound = ACC_REL * (_chunk_max(dod[rows, h]) @ _chunk_max(vd[keys, h // grp]).T + np.abs(Dr)) + \
            2.0 ** -22 * np.abs(ex)
        for y, got in enumerate((DP[x].astype(np.float64) * np.exp2(edo[x] - eq[x]), -DQP[x].astype(np.float64))):
            err = np.where(vis, np.abs(got - ex), 0.0)
            worst[y] = max(worst[y], float((err / np.where(vis, bound, 1.0)).max()))
            assert (err <= bound).all(), "D - dP beyond the accumulation bound"
    say("  D - dP vs exact dot products: key-tile pass (unfolded) max error / bound %.3f, dQ pass %.3f"
        % tuple(worst))
    # the dQ pass's scores: bit-identical to the key-tile pass's, masks included
    S = du["bwd_s"]
    assert np.array_equal(np.isnan(S), np.isnan(du["dq_s"])), "dQ pass: pairs visited"
    assert np.array_equal(S.view(np.uint32), du["dq_s"].view(np.uint32)), "dQ pass: scores"
    say("  dQ pass scores: bit-identical to the key-tile pass's (%d pairs)" % int((~np.isnan(S)).sum()))
    # 4'. decisions: P'' and dS'' (32 x 32 blocks), dS' (per row and 32-key block)
    lse = np.stack([g["lse"][h, rows] for h in hs])[:, :, None]
    ek = np.stack([g["sk"][h // grp, keys] for h in hs]).astype(np.float64)[:, None, :] - 127
    with np.errstate(invalid="ignore", over="ignore"):
        Pv = np.exp2(fma32(S, c32, -lse).astype(np.float64)).astype(np.float32)
        P2 = (Pv.astype(np.float64) * np.exp2(edo)).astype(np.float32)
        dS2 = -(P2.astype(np.float64) * DP.astype(np.float64)).astype(np.float32)
        dS0 = (Pv.astype(np.float64) * DQP.astype(np.float64)).astype(np.float32)
        dS1 = dS0.astype(np.float64) * np.exp2(ek)
        # values below FP32's normal range at some step of their formation (the exponential, the
        # fold, the product, the converted value)
        sub = lambda x: np.abs(x) < 2.0 ** -126
        tiny = dict(p=sub(Pv) | sub(P2), ds=sub(Pv) | sub(P2) | sub(dS2), dsq=sub(Pv) | sub(dS0) | sub(dS1))
    vis3 = np.broadcast_to(vis, S.shape)
    vals = dict(p=np.where(vis3, P2, 0.0).astype(np.float64), ds=np.where(vis3, dS2, 0.0).astype(np.float64),
                dsq=np.where(vis3, dS1, 0.0))
    dm = doc_map(cu, T)
    counts = dict(p=[0, 0, 0], ds=[0, 0, 0], dsq=[0, 0, 0], tiny=0)
    for doc in sorted(set(dm[win["row_lo"]:win["row_hi"]]) - {-1}):
        a, b = int(cu[doc]), int(cu[doc + 1])
        r0, r1 = max(a, win["row_lo"]), min(b, win["row_hi"])
        assert (r0 - a) % 32 == 0, "window rows must start on a block of the document"
        rs, ks = slice(r0 - win["row_lo"], r1 - win["row_lo"]), slice(a - win["key_lo"], b - win["key_lo"])
        v_doc = np.broadcast_to(vis[rs, ks], (len(hs),) + vis[rs, ks].shape)
        for nm, code, ex in (("p", du["bwd_p"], du["bwd_ps"]), ("ds", du["bwd_ds"], du["bwd_dss"]),
                             ("dsq", du["dq_ds"], du["dq_dss"])):
            label = {"p": "P''", "ds": "dS''", "dsq": "dS'"}[nm]
            if nm == "dsq":
                counts[nm][2] += check_row_exponents(label, ex[:, rs, ks], vals[nm][:, rs, ks], v_doc, orc)
            else:
                counts[nm][2] += check_block_exponents(label, ex[:, rs, ks], vals[nm][:, rs, ks], v_doc, orc)
            y = np.where(v_doc, vals[nm][:, rs, ks] * np.exp2(127.0 - ex[:, rs, ks].astype(np.float64)), 0.0)
            # the hardware returns +0 for values below FP32's normal range (the exponential's result,
            # a denormal input of the conversion), where the method's value is a tiny nonzero
            # number; with per-token exponents folded in (and one exponent per row for dS') such a
            # value can still reach E4M3 resolution.  A zero code is accepted there: the term is
            # below 2^-126 times an operand of the product, far under the FP32 sums' rounding and,
            # for dQ, under the FP16 sums' smallest value (|x 2^pi| < 2^-62)
            lo_ok = tiny[nm][:, rs, ks] & (orc.e4m3_decode(code[:, rs, ks]) == 0)
            counts["tiny"] += int((lo_ok & v_doc & (orc.e4m3_decode(orc.e4m3_rne(y)) != 0)).sum())
            nb, nt = check_decision(label + " codes", code[:, rs, ks], y, orc, v_doc, lo_ok=lo_ok)
            counts[nm][0] += nb
            counts[nm][1] += nt
    if counts["tiny"]:
        say("  %d codes zero where a value on the way is below FP32's normal range (accepted)"
            % counts["tiny"])
    for nm, label in (("p", "P''"), ("ds", "dS''"), ("dsq", "dS'")):
        say("  %-4s: %d / %d codes and %d exponents at a rounding boundary, the rest equal the oracle's rounding"
            % (label, counts[nm][0], counts[nm][1], counts[nm][2]))
    # 5'. products against the replays on the GPU's decisions (operands with bare codes where their
    # exponent was folded into the other one)
    bare = lambda t: np.full_like(t, 127)
    r = orc.bwd_replay(g["q"], bare(g["sq"]), g["k"], g["sk"], g["do"], bare(g["sdo"]), cu, pi, win, du["bwd_p"],
                       du["bwd_ps"], du["bwd_ds"], du["bwd_dss"], ss)
    rq = orc.bwd_replay(g["q"], g["sq"], g["k"], bare(g["sk"]), g["do"], g["sdo"], cu, pi, win, du["bwd_p"],
                        du["bwd_ps"], du["dq_ds"], du["dq_dss"], ss)
    r["dq64"] = rq["dq64"]
    rmask = dm[win["row_lo"]:win["row_hi"]] >= 0
    got_dq = np.transpose(g["dq"][rows][:, win["head_lo"]:win["head_hi"]], (1, 0, 2))
    dq16 = validate_dq_partials(orc, g, cu, pi, ss, ds_name="dq_ds", k_bare=True)
    same = np.array_equal(got_dq[:, rmask], dq16[:, rmask])
    say("  stage dQ vs the FP16 sum of the GPU's partials (ascending tiles, two roundings each): bit-identical %s"
        % same)
    assert same, "dQ"
    beyond = {"dQ": bar_check("dQ", got_dq[:, rmask], r["dq64"][:, rmask], orc, enforce=False)}
    kv = [x for x in range(Hkv) if x * grp >= win["head_lo"] and (x + 1) * grp <= win["head_hi"]]
    kmask = rmask & ~np.isnan(r["dk64"][kv[0], :, 0]) if kv else rmask
    for nm, ref in (("dK", r["dk64"]), ("dV", r["dv64"])):
        got = np.transpose(g[nm.lower()][rows][:, kv], (1, 0, 2))
        beyond[nm] = bar_check(nm, got[:, kmask], ref[kv][:, kmask], orc)
    return dict(replay=r, kv=kv, kmask=kmask, beyond=beyond, dq16=dq16)


def chain_check(orc, g, ref, cu, fwd_val, bwd_val, zero_in_exact=()):
    """The whole GPU call against the oracle's own chain on the BF16 inputs (window rows and
    heads): codes, scales, pi bit-exact; cosine >= 0.9995 per tensor; every element beyond
    2e-2 RMS + one BF16 ulp named with the part of its difference that the GPU's validated
    decisions account for (replay minus oracle).  zero_in_exact: outputs that vanish in exact
    arithmetic (rounding-level values: cosine undefined, not gated)."""
    win = g["window"]
    for nm in ("q", "sq", "k", "sk", "v", "sv", "do", "sdo", "pi") + (("q4", "sq4", "k4", "sk4") if g.get("qk4") else ()):
        assert np.array_equal(g[nm], ref[nm]), nm
    T = g["q"].shape[0]
    dm = doc_map(cu, T)
    rows = slice(win["row_lo"], win["row_hi"])
    rmask = dm[rows] >= 0
    hs = slice(win["head_lo"], win["head_hi"])
    kv, kmask = bwd_val["kv"], bwd_val["kmask"]
    items = [("O", g["o"][rows][rmask][:, hs], ref["o"][rows][rmask][:, hs],
              np.transpose(fwd_val["o64"], (1, 0, 2))[rmask]),
             ("dQ", g["dq"][rows][rmask][:, hs], ref["dq"][rows][rmask][:, hs],
              bits_to_f64(np.transpose(bwd_val["dq16"], (1, 0, 2))[rmask]))]
    if kv:
        items += [("dK", g["dk"][rows][kmask][:, kv], ref["dk"][rows][kmask][:, kv],
                   np.transpose(bwd_val["replay"]["dk64"][kv], (1, 0, 2))[kmask]),
                  ("dV", g["dv"][rows][kmask][:, kv], ref["dv"][rows][kmask][:, kv],
                   np.transpose(bwd_val["replay"]["dv64"][kv], (1, 0, 2))[kmask])]
    for nm, gb, rb, rep in items:
        if not gb.size:
            say("  chain %-3s: no rows in the window (non-causal keys outside a document-start window)" % nm)
            continue
        gv, rv = bits_to_f64(gb), bits_to_f64(rb)
        repv = bits_to_f64(orc.bf16_rne(rep))
        c = cosine(gv, rv)
        scale = rms(rv)
        diff = np.abs(gv - rv)
        bar = MAXABS_REL * scale + bf16_ulp(rv)
        beyond = np.nonzero(diff > bar)
        decided = np.abs(repv - rv)
        say("  chain %-3s vs oracle: cosine %.7f  max|diff|/rms %.3e  beyond 2e-2 rms + 1 ulp: %d/%d"
            % (nm, c, diff.max() / max(scale, 1e-300), len(beyond[0]), gv.size))
        for t in range(min(len(beyond[0]), 8)):
            ix = tuple(a[t] for a in beyond)
            say("    %s%s: |gpu - oracle| %.3e rms, of which the GPU's decisions (replay - oracle) %.3e rms, "
                "GPU vs replay %.3e rms" % (nm, ix, diff[ix] / scale, decided[ix] / scale,
                                            abs(gv[ix] - repv[ix]) / scale))
        # the excess over the bar is what the decisions account for: |gpu - replay| meets the bar
        assert (np.abs(gv - repv)[beyond] <= (MAXABS_REL * scale + bf16_ulp(repv))[beyond]).all(), nm
        if nm not in zero_in_exact:
            assert c >= COS_MIN, (nm, c)


def check_cosine(name, got_bits, ref_bits, mask=None):
    """End-to-end cosine (north star bar >= 0.9995, FP64) with max-abs reported."""
    g, r = bits_to_f64(got_bits), bits_to_f64(ref_bits)
    if mask is not None:
        g, r = g[mask], r[mask]
    if not g.size:
        return
    c = cosine(g, r)
    scale = rms(r)
    say("  chain %-3s cosine %.7f  max|diff|/rms %.3e" % (name, c, np.abs(g - r).max() / scale))
    assert c >= COS_MIN, (name, c)


def full_window(T, Hq):
    return dict(row_lo=0, row_hi=T, key_lo=0, key_hi=T, head_lo=0, head_hi=Hq)


def doc_window(cu, doc, heads, tail_blocks=0):
    """Rows of one document (its last tail_blocks 32-query blocks, or all), all its keys."""
    a, b = int(cu[doc]), int(cu[doc + 1])
    nb = -(-(b - a) // 32)
    r0 = a + 32 * max(nb - tail_blocks, 0) if tail_blocks else a
    return dict(row_lo=r0, row_hi=b, key_lo=a, key_hi=b, head_lo=heads[0], head_hi=heads[1])


def stage_and_chain(orc, q, k, v, do, cu, window, causal_dq=False, release=None, tail=False, zero_in_exact=(),
                    causal=True, hadamard=False, qk4=False):
    """Debug run in `window` (compared bit for bit with the product library's run `release`, made
    here if not given), decision checks and replays (stage), then the oracle's own chain (its
    work restricted to the window's documents, KV heads and, with tail=True, document tail)."""
    cu = np.asarray(cu, np.int32)
    if release is None:
        release = gpu_call(q, k, v, do, cu, causal_dq, causal=causal, hadamard=hadamard, qk4=qk4)
    g = gpu_call(q, k, v, do, cu, causal_dq, window=window, causal=causal, hadamard=hadamard, qk4=qk4)
    same_outputs(g, release)
    say("  debug variant: outputs bit-identical to libflamia.so")
    fv = validate_forward(orc, g, cu)
    bv = validate_backward(orc, g, cu, causal_dq)
    T, Hq = g["q"].shape[:2]
    grp = Hq // g["k"].shape[1]
    kvh = list(range(window["head_lo"] // grp, -(-window["head_hi"] // grp)))
    docs = sorted(set(doc_map(cu, T)[window["row_lo"]:window["row_hi"]]) - {-1})
    kw = dict(docs=docs if len(docs) < len(cu) - 1 else None,
              kv_heads=kvh if len(kvh) < g["k"].shape[1] else None)
    if tail:
        tr = window["row_hi"] - window["row_lo"]
        kw.update(tail_rows=tr, tail_blocks=-(-tr // 32))
    ref = oracle_call(orc, q, k, v, do, cu, causal_dq, causal=causal, hadamard=hadamard, qk4=qk4, **kw)
    if hadamard:  # the GPU run above returns dQ, dK in the rotated basis
        ref["dq"], ref["dk"] = ref["dq_rot"], ref["dk_rot"]
    chain_check(orc, g, ref, cu, fv, bv, zero_in_exact)
    return g


def token_mask(cu, T, docs=None):
    m = np.zeros(T, bool)
    cu = np.asarray(cu)
    for i, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        if docs is None or i in docs:
            m[a:b] = True
    return m
