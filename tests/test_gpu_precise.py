"""GPU parity of the precision options (jaehun.me §3.2, §4.5; per-token operand scales, V folded
into the probability operand) against the oracle, through the C ABI: per-token codes, scales and
D bit-exact; every probability code of the precise forward equal to the oracle's rounding of its
definition (or at a rounding boundary); O and LSE against the oracle's replay on the GPU's
decisions and against the oracle's own chain; and no leakage: perturbing a document from inside
a 32-token block leaves every earlier row's O and LSE bit-identical."""
import ctypes

import numpy as np
import pytest
import torch

import precision_causal_attention_token_amd as fl
from precision_causal_attention_token_amd import workloads
from tests import gpu_common as gc
from tests.helpers import bf16_bits, bits_to_f64, cosine

pytestmark = pytest.mark.gpu


def _quant(xs, cu_d):
    out = fl.quantize([x.cuda() for x in xs], cu_d, per_token=True)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("d", [64, 128])
def test_per_token_quantiser_bit_exact(orc, d):
    T, Hq, Hkv = 1200, 4, 2
    cu = np.array([9, 40, 41, 555, 555, 1100], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=1400 + d, outlier_channels=2)
    cu_d = torch.as_tensor(cu).cuda()
    out = _quant([q, k, v], cu_d)
    for (c, s), x in zip(out, (q, k, v)):
        rc, rs = orc.quantize(bf16_bits(x), cu, per_token=True)
        assert np.array_equal(c.cpu().numpy(), rc) and np.array_equal(s.cpu().numpy(), rs)
    o = torch.randn(T, Hq, d).to(torch.bfloat16)
    dc, dsc, D = fl.quantize_do(do.cuda(), o.cuda(), cu_d, per_token=True)
    rc, rs, rD = orc.quantize_do(bf16_bits(do), bf16_bits(o), cu, per_token=True)
    assert np.array_equal(dc.cpu().numpy(), rc) and np.array_equal(dsc.cpu().numpy(), rs)
    gD = D.cpu().numpy()
    assert np.abs(gD - rD).max() <= 1e-5 * max(np.abs(rD).max(), 1e-30)
    gc.say("  per-token quantiser d=%d: codes and scales bit-exact, D within 1e-5" % d)


def _wshape(w):
    return (w["head_hi"] - w["head_lo"], w["row_hi"] - w["row_lo"], w["key_hi"] - w["key_lo"])


def _fwd(q, k, v, cu, window=None):
    """Per-token quantisation and the precise forward; with `window` the debug library's dumps."""
    cu_d = torch.as_tensor(np.asarray(cu, np.int32)).cuda()
    T = q.shape[0]
    lib = gc.debug_library() if window is not None else fl.load_library()
    bufs = None
    with gc.using(lib):
        if window is not None:
            shp = _wshape(window)
            bufs = {n: torch.full(shp, float("nan"), dtype=torch.float32, device="cuda") for n in gc.DUMP_F32}
            bufs.update({n: torch.full(shp, 0xFF, dtype=torch.uint8, device="cuda") for n in gc.DUMP_U8})
            bufs["dq_part"] = torch.full(shp[:2] + (1, q.shape[2]), float("nan"), dtype=torch.float32, device="cuda")
            assert lib.flamia_debug_set_dump(ctypes.byref(gc._dump_struct(window, bufs))) == 0
        try:
            lists = fl.Lists(cu_d, T)
            qz, kz, vz = fl.quantize([q.cuda(), k.cuda(), v.cuda()], cu_d, per_token=True)
            o, lse = fl.fwd(qz, kz, vz, cu_d, lists.fwd, precise=True)
            torch.cuda.synchronize()
        finally:
            if window is not None:
                lib.flamia_debug_set_dump(None)
    n = lambda t: t.cpu().numpy()
    out = dict(q=n(qz[0]), sq=n(qz[1]), k=n(kz[0]), sk=n(kz[1]), v=n(vz[0]), sv=n(vz[1]),
               o=bf16_bits(o.cpu()), lse=n(lse))
    if bufs is not None:
        out["dumps"] = {k_: n(t) for k_, t in bufs.items()}
    return out


def _vref(sv, cu, win, grp, Hq):
    """[heads][rows][keys] of the window: the V exponent reference of each (row, key) pair's tile:
    the running maximum over the row's visible keys of the tiles visited up to it (diagonal tile
    first), at least -119."""
    T = sv.shape[1]
    nh, nr, nk = _wshape(win)
    out = np.full((nh, nr, nk), -1000, np.int64)
    for doc, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        for hx, h in enumerate(range(win["head_lo"], win["head_hi"])):
            e = sv[h // grp, a:b].astype(np.int64) - 127
            for r in range(max(a, win["row_lo"]), min(b, win["row_hi"])):
                ref = -119
                i = r - a
                for kt in range(i // 128, -1, -1):
                    j0, j1 = 128 * kt, min(128 * kt + 128, i + 1)
                    ref = max(ref, int(e[j0:j1].max()))
                    out[hx, r - win["row_lo"], a + j0 - win["key_lo"]:a + j1 - win["key_lo"]] = ref
    return out


def _validate_fwd(orc, g, cu):
    """The precise forward's decisions and products: every probability code equal to the oracle's
    rounding of 2^(fma(S, c, 8 - m) + e(V_j) - v_i) (or at a rounding boundary), O and LSE against
    the oracle's replay on the GPU's decisions.  Returns dict(o64) for the chain check."""
    win, du = g["window"], g["dumps"]
    T, Hq, d = g["q"].shape
    Hkv = g["k"].shape[1]
    c32 = gc.score_scale32(d)
    vis = gc.visible_mask(cu, T, win)
    S, M, P = du["fwd_s"], du["fwd_m"], du["fwd_p"]
    grp = Hq // Hkv
    ref = _vref(g["sv"], cu, win, grp, Hq)
    ekey = np.stack([np.broadcast_to((g["sv"][h // grp].astype(np.int64) - 127)[None, :], (T, T)) for h in range(Hq)])
    ekey = ekey[win["head_lo"]:win["head_hi"], win["row_lo"]:win["row_hi"], win["key_lo"]:win["key_hi"]]
    with np.errstate(invalid="ignore", over="ignore"):
        y = np.exp2(gc.fma32(S, c32, (np.float32(8) - M).astype(np.float32)).astype(np.float64))
        y = y * np.exp2((ekey - ref).astype(np.float64))
    v3 = np.broadcast_to(vis, y.shape)
    y = np.where(v3, y, 0.0)
    nb, nt = gc.check_decision("precise probability codes", P, y, orc, v3)
    gc.say("  probability codes: %d / %d at a rounding boundary, the rest equal the oracle's rounding" % (nb, nt))
    o64, lse64 = orc.fwd_replay(g["v"], g["sv"], cu, win, S.astype(np.float64), M.astype(np.float64), P, Hq,
                                float(c32), precise=True)
    rmask = gc.doc_map(cu, T) >= 0
    got_o = np.transpose(g["o"], (1, 0, 2))
    gc.bar_check("O", got_o[:, rmask], o64[:, rmask], orc)
    lerr = np.abs(g["lse"][:, rmask].astype(np.float64) - lse64[:, rmask])
    assert lerr.max() <= 1e-4, lerr.max()
    return dict(o64=o64)


@pytest.mark.parametrize("name,T,Hq,Hkv,d,cu", [
    ("packed-d128", 1100, 4, 2, 128, [0, 300, 301, 700, 1100]),
    ("offsets-d64", 1200, 4, 1, 64, [9, 40, 41, 555, 555, 1100]),
])
def test_precise_forward_parity(orc, name, T, Hq, Hkv, d, cu):
    gc.say("precise forward %s" % name)
    q, k, v, _ = workloads.tensors(T, Hq, Hkv, d, seed=1420, outlier_channels=2)
    cu = np.asarray(cu, np.int32)
    win = gc.full_window(T, Hq)
    rel = _fwd(q, k, v, cu)
    g = _fwd(q, k, v, cu, window=win)
    g["window"] = win
    assert np.array_equal(g["o"], rel["o"]) and np.array_equal(g["lse"].view(np.uint32), rel["lse"].view(np.uint32))
    _validate_fwd(orc, g, cu)
    # the oracle's own chain on the BF16 inputs
    r = {}
    for nm, x in (("q", q), ("k", k), ("v", v)):
        r[nm], r["s" + nm] = orc.quantize(bf16_bits(x), cu, per_token=True)
    ro, rl, _ = orc.fwd(r["q"], r["sq"], r["k"], r["sk"], r["v"], r["sv"], cu, precise=True)
    rmask = gc.doc_map(cu, T) >= 0
    c = cosine(bits_to_f64(g["o"][rmask]), bits_to_f64(ro[rmask]))
    gc.say("  chain O vs oracle: cosine %.7f" % c)
    assert c >= gc.COS_MIN


@pytest.mark.parametrize("p", [37, 161])
def test_precise_forward_no_leakage(p):
    """Q, K, V perturbed (x16) from offset p (inside a 32-token block) to the document end: the
    precise forward's O and LSE of every earlier row and of the other document are
    bit-identical."""
    T, Hq, Hkv, d = 520, 4, 2, 128
    cu = np.array([0, 300, T], np.int32)
    q, k, v, _ = workloads.tensors(T, Hq, Hkv, d, seed=1430)
    keep = np.ones(T, bool)
    keep[p:300] = False
    runs = []
    for scale in (1.0, 16.0):
        xs = []
        for x in (q, k, v):
            y = x.clone()
            y[p:300] = (y[p:300].to(torch.float32) * scale).to(torch.bfloat16)
            xs.append(y)
        runs.append(_fwd(*xs, cu))
    a, b = runs
    assert not np.array_equal(a["o"], b["o"])
    assert np.array_equal(a["o"][keep], b["o"][keep])
    assert np.array_equal(a["lse"][:, keep].view(np.uint32), b["lse"][:, keep].view(np.uint32))
    gc.say("  precise forward, perturbation from offset %d: earlier rows bit-identical" % p)


# ------------------------------------------------------------------------------------------
# Backward under the precision options: dK, dV from the key-tile pass with dO's exponent folded
# into P and Q's into dS, dQ from the query-stationary pass with K's exponent folded into dS and
# one dS exponent per (query row, 32-key block).

def _train(q, k, v, do, cu, precise=True, store_budget=None, static_scratch=False, window=None):
    """The whole GPU call (per-token quantisation, forward, dO pass, backward) with the precision
    options, or the default one; numpy outputs, BF16 as bit patterns.  With `window` the debug
    variant runs and its per-pair dumps come back under "dumps"."""
    cu_d = torch.as_tensor(np.asarray(cu, np.int32)).cuda()
    T, Hq, d = q.shape
    lib = gc.debug_library() if window is not None else fl.load_library()
    bufs = None
    with gc.using(lib):
        if window is not None:
            shp = _wshape(window)
            bufs = {n: torch.full(shp, float("nan"), dtype=torch.float32, device="cuda") for n in gc.DUMP_F32}
            bufs.update({n: torch.full(shp, 0xFF, dtype=torch.uint8, device="cuda") for n in gc.DUMP_U8})
            bufs["dq_part"] = torch.full(shp[:2] + (gc.n_key_tiles(window), d), float("nan"), dtype=torch.float32,
                                         device="cuda")
            assert lib.flamia_debug_set_dump(ctypes.byref(gc._dump_struct(window, bufs))) == 0
        try:
            lists = fl.Lists(cu_d, T)
            qz, kz, vz = fl.quantize([q.cuda(), k.cuda(), v.cuda()], cu_d, per_token=precise)
            o, lse = fl.fwd(qz, kz, vz, cu_d, lists.fwd, precise=precise)
            dc, dsc, D = fl.quantize_do(do.cuda(), o, cu_d, per_token=precise)
            kw = dict(want_pi=True, precise=precise)
            if static_scratch:
                kw["static_scratch"] = True
            else:
                budget = fl.DEFAULT_STORE_BYTES if store_budget is None else store_budget
                kw["workspace"] = torch.empty(fl.bwd_workspace_bytes(len(cu) - 1, T, Hq, d, budget),
                                              dtype=torch.uint8, device="cuda").fill_(0xA5)
            dq, dk, dv, pi = fl.bwd(qz, kz, vz, (dc, dsc), lse, D, cu_d, lists, **kw)
            torch.cuda.synchronize()
        finally:
            if window is not None:
                lib.flamia_debug_set_dump(None)
    n = lambda t: t.cpu().numpy()
    b = lambda t: bf16_bits(t.cpu())
    out = dict(q=n(qz[0]), sq=n(qz[1]), k=n(kz[0]), sk=n(kz[1]), v=n(vz[0]), sv=n(vz[1]), do=n(dc), sdo=n(dsc),
               D=n(D), o=b(o), lse=n(lse), dq=b(dq), dk=b(dk), dv=b(dv), pi=n(pi), causal=True)
    if bufs is not None:
        out["dumps"] = {k_: n(t) for k_, t in bufs.items()}
        out["window"] = dict(window)
    return out


@pytest.mark.parametrize("name,T,Hq,Hkv,d,cu", [
    ("packed-d128", 1100, 4, 2, 128, [0, 300, 301, 700, 1100]),
    ("offsets-d64", 1200, 4, 1, 64, [9, 40, 41, 555, 555, 1100]),
    ("one-tile-docs-d128", 700, 2, 2, 128, [0, 1, 33, 128, 200, 329, 457, 700]),
])
def test_precise_backward_parity(orc, name, T, Hq, Hkv, d, cu):
    """Stage: the debug variant (outputs bit-identical to the product library's) and every
    decision of the precise backward checked against the oracle's rounding of its definition,
    dQ, dK, dV against the oracle's replays on those decisions.  Chain: the whole call against
    the oracle's own precise chain on the BF16 inputs (codes, scales, pi bit-exact; cosine >=
    0.9995; every element beyond 2e-2 RMS + 1 ulp accounted for by the GPU's validated
    decisions)."""
    gc.say("precise backward %s" % name)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=1440, outlier_channels=2)
    cu = np.asarray(cu, np.int32)
    rel = _train(q, k, v, do, cu)
    g = _train(q, k, v, do, cu, window=gc.full_window(T, Hq))
    gc.same_outputs(g, rel)
    gc.say("  debug variant: outputs bit-identical to libflamia.so")
    rows = gc.doc_map(cu, T) >= 0
    for nm in ("dq", "dk", "dv"):
        assert not g[nm][~rows].any(), nm              # rows outside every document: zero
    fv = _validate_fwd(orc, g, cu)
    bv = gc.validate_backward_precise(orc, g, cu)
    # the oracle's own chain on the BF16 inputs
    r = {}
    for nm, x in (("q", q), ("k", k), ("v", v)):
        r[nm], r["s" + nm] = orc.quantize(bf16_bits(x), cu, per_token=True)
    ro, rl, _ = orc.fwd(r["q"], r["sq"], r["k"], r["sk"], r["v"], r["sv"], cu, precise=True)
    dc, dsc, D = orc.quantize_do(bf16_bits(do), ro, cu, per_token=True)
    rg = orc.bwd(r["q"], r["sq"], r["k"], r["sk"], r["v"], r["sv"], dc, dsc, rl, D, cu, precise=True)
    r.update(do=dc, sdo=dsc, D=D, o=ro, lse=rl, dq=rg["dq"], dk=rg["dk"], dv=rg["dv"], pi=rg["pi"])
    gc.chain_check(orc, g, r, cu, fv, bv)


def test_precise_backward_workspace_and_static_scratch_identical():
    """One chunk whatever the workspace (nothing is stored): the smallest workspace and the
    static-scratch entry point give the same bits as the default workspace."""
    T, Hq, Hkv, d = 900, 4, 2, 128
    cu = np.array([0, 600, 601, 900], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=1441)
    a = _train(q, k, v, do, cu)
    for kw in (dict(store_budget=0), dict(static_scratch=True)):
        b = _train(q, k, v, do, cu, **kw)
        for nm in ("dq", "dk", "dv", "pi"):
            assert np.array_equal(a[nm], b[nm]), (kw, nm)
    gc.say("  precise backward: smallest workspace and static scratch bit-identical to the default")


@pytest.mark.parametrize("p", [37, 161, 290])
def test_precise_backward_no_leakage(p):
    """Q, K, V perturbed (x16) from offset p (inside a 32-token block) to the end of document 0
    and dO zero there (the loss does not see those rows): with the precision options dQ of every
    earlier row and dK, dV of every earlier key, and everything of the other document, are
    bit-identical; the default scales' dK / dV are not (the probe is sensitive)."""
    T, Hq, Hkv, d = 520, 4, 2, 128
    cu = np.array([0, 300, T], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=1442, outlier_channels=2)
    do = do.clone()
    do[p:300] = 0
    keep = np.ones(T, bool)
    keep[p:300] = False
    res = {}
    for precise in (True, False):
        runs = []
        for scale in (1.0, 16.0):
            xs = []
            for x in (q, k, v):
                y = x.clone()
                y[p:300] = (y[p:300].to(torch.float32) * scale).to(torch.bfloat16)
                xs.append(y)
            runs.append(_train(*xs, do, cu, precise=precise))
        res[precise] = runs
    for run in res[True] + res[False]:
        for nm in ("o", "dq", "dk", "dv"):
            assert np.isfinite(bits_to_f64(run[nm])).all(), nm
    a, b = res[True]
    assert not np.array_equal(a["o"], b["o"])           # the perturbation took effect
    for nm in ("dq", "dk", "dv"):
        assert np.array_equal(a[nm][keep], b[nm][keep]), nm
    a0, b0 = res[False]
    leaks = [nm for nm in ("dq", "dk", "dv") if not np.array_equal(a0[nm][keep], b0[nm][keep])]
    gc.say("  precise backward, perturbation from offset %d: earlier dQ, dK, dV bit-identical "
           "(default scales differ in: %s)" % (p, ", ".join(leaks) or "none"))
    if p % 32:
        assert "dk" in leaks                            # Q's block scale reaches earlier keys' dK


@pytest.mark.parametrize("p", [37, 290])
def test_precise_dq_no_leakage_with_live_gradients(p):
    """Q, K, V and dO all perturbed (x16) from offset p to the end of document 0 (dO too, so the
    later rows' dS, its exponents and pi are all live and changed): with the precision options
    dQ of every earlier row, and O, LSE, D, is bit-identical."""
    T, Hq, Hkv, d = 520, 4, 2, 64
    cu = np.array([0, 300, T], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=1443, outlier_channels=2)
    keep = np.ones(T, bool)
    keep[p:300] = False
    runs = []
    for scale in (1.0, 16.0):
        xs = []
        for x in (q, k, v, do):
            y = x.clone()
            y[p:300] = (y[p:300].to(torch.float32) * scale).to(torch.bfloat16)
            xs.append(y)
        runs.append(_train(*xs, cu))
    a, b = runs
    for run in runs:
        for nm in ("o", "dq", "dk", "dv"):
            assert np.isfinite(bits_to_f64(run[nm])).all(), nm
    assert not np.array_equal(a["dq"], b["dq"])
    assert np.array_equal(a["dq"][keep], b["dq"][keep])
    assert np.array_equal(a["o"][keep], b["o"][keep])
    for nm in ("lse", "D"):
        assert np.array_equal(a[nm][:, keep].view(np.uint32), b[nm][:, keep].view(np.uint32)), nm
    gc.say("  precise dQ, live perturbation from offset %d: earlier rows bit-identical" % p)
