"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI and the oracle on
the same seeded inputs, and compare them at the acceptance bar:
  codes, scales, pi, work lists: bit-exact;
  O, dQ, dK, dV: cosine >= 0.9995 and max |diff| <= 2e-2 * RMS(oracle), per tensor, FP64."""
import sys

import numpy as np
import torch

import precision_causal_attention_token_amd as fl
from tests.helpers import bf16_bits, bits_to_f64, cosine, rms

COS_MIN = 0.9995
MAXABS_REL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_gpu(*xs):
    return [torch.as_tensor(x).cuda() for x in xs]


def gpu_call(q, k, v, do, cu, causal_dq=False, softmax_scale=None):
    """Full training call on the GPU; returns numpy arrays (BF16 outputs as bit patterns)."""
    dev = torch.device("cuda:0")
    cu_d = torch.as_tensor(np.asarray(cu, np.int32)).to(dev)
    T = q.shape[0]
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    lists = fl.Lists(cu_d, T)
    qz, kz, vz = fl.quantize([qd, kd, vd], cu_d)
    o, lse = fl.fwd(qz, kz, vz, cu_d, lists.fwd, softmax_scale)
    dc, dsc, D = fl.quantize_do(dod, o, cu_d)
    Hq = q.shape[1]
    ws = torch.empty(fl.bwd_workspace_bytes(cu, T, Hq), dtype=torch.uint8, device=dev)
    ws.fill_(0xA5)  # the workspace may hold anything on entry
    dq, dk, dv, pi = fl.bwd(qz, kz, vz, (dc, dsc), lse, D, cu_d, lists, softmax_scale, causal_dq, want_pi=True,
                            workspace=ws)
    torch.cuda.synchronize()
    assert fl.bwd_status(ws) == 0, 'backward workspace status'
    b = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
    n = lambda t: t.cpu().numpy()
    return dict(q=n(qz[0]), sq=n(qz[1]), k=n(kz[0]), sk=n(kz[1]), v=n(vz[0]), sv=n(vz[1]),
                do=n(dc), sdo=n(dsc), D=n(D), o=b(o), lse=n(lse), dq=b(dq), dk=b(dk), dv=b(dv), pi=n(pi))


def oracle_call(orc, q, k, v, do, cu, causal_dq=False, softmax_scale=None, docs=None, kv_heads=None):
    """The oracle's own end-to-end chain on the BF16 inputs."""
    cu = np.asarray(cu, np.int32)
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        c, s = orc.quantize(bf16_bits(x), cu)
        out[name], out["s" + name] = c, s
    o, lse, _ = orc.fwd(out["q"], out["sq"], out["k"], out["sk"], out["v"], out["sv"], cu, softmax_scale,
                        docs=docs, kv_heads=kv_heads)
    dc, dsc, D = orc.quantize_do(bf16_bits(do), o, cu)
    g = orc.bwd(out["q"], out["sq"], out["k"], out["sk"], out["v"], out["sv"], dc, dsc, lse, D, cu, softmax_scale,
                causal_dq=causal_dq, docs=docs, kv_heads=kv_heads)
    out.update(do=dc, sdo=dsc, D=D, o=o, lse=lse, dq=g["dq"], dk=g["dk"], dv=g["dv"], pi=g["pi"])
    return out


def check_cosine(name, got_bits, ref_bits, mask=None):
    """End-to-end bar (the benchmark spec): cosine >= 0.9995 per tensor, FP64; max-abs reported."""
    g, r = bits_to_f64(got_bits), bits_to_f64(ref_bits)
    if mask is not None:
        g, r = g[mask], r[mask]
    if not g.size:
        return
    c = cosine(g, r)
    scale = rms(r)
    say("  chain %-3s cosine %.7f  max|diff|/rms %.3e" % (name, c, np.abs(g - r).max() / scale))
    assert c >= COS_MIN, (name, c)


def assert_close(name, got_bits, ref_bits, flip, acc, mask=None, need_cosine=True):
    """Stage bar, on BF16 bit patterns: cosine >= 0.9995 (per tensor, FP64) and per element
      |gpu - oracle| <= 2e-2 * RMS(oracle) + one BF16 ulp of the oracle value + flip + acc.
    flip: the oracle's one-flip allowance (largest change one E4M3 code of a computed operand,
    Phat or dShat, moving to its neighbour causes in that element); acc: the oracle's first-
    order bound of the FP8 matrix instruction's accumulation error.  Both, and the ulp, come
    from the arithmetic (see the oracle's allowance function)."""
    g, r = bits_to_f64(got_bits), bits_to_f64(ref_bits)
    F = np.asarray(flip, np.float64)
    A = np.asarray(acc, np.float64)
    if mask is not None:
        g, r, F, A = g[mask], r[mask], F[mask], A[mask]
    if not g.size:
        return
    c = cosine(g, r)
    diff = np.abs(g - r)
    scale = rms(r)
    bound = MAXABS_REL * scale + bf16_ulp(r) + F + A
    excess = (diff - bound).max()
    say("  stage %-3s cosine %.7f  max|diff|/rms %.3e  beyond 2e-2 rms: %d/%d  worst margin %.3e rms  "
        "(median allowance %.2e rms)" % (name, c, diff.max() / scale, int((diff > MAXABS_REL * scale).sum()),
                                         diff.size, -excess / scale, float(np.median(F + A)) / scale))
    if need_cosine:
        assert c >= COS_MIN, (name, c)
    assert excess <= 0, (name, excess / scale)


def stage_check(orc, g, cu, causal_dq=False, softmax_scale=None, docs=None, kv_heads=None, q_heads=None,
                zero_in_exact=()):
    """zero_in_exact: outputs that vanish in exact arithmetic (cosine undefined; only the
    per-element bound applies)."""
    """Forward stage against the oracle's forward on the GPU's (bit-exact) codes; backward stage
    against the oracle's backward on the same codes and the GPU's own LSE and D."""
    cu = np.asarray(cu, np.int32)
    T = g["q"].shape[0]
    o, lse, o64, oflip = orc.fwd(g["q"], g["sq"], g["k"], g["sk"], g["v"], g["sv"], cu, softmax_scale,
                                 want_o64=True, want_flip=True, docs=docs, kv_heads=kv_heads)
    r = orc.bwd(g["q"], g["sq"], g["k"], g["sk"], g["v"], g["sv"], g["do"], g["sdo"], g["lse"], g["D"], cu,
                softmax_scale, causal_dq=causal_dq, want_flip=True, docs=docs, kv_heads=kv_heads)
    A = orc.allowance(g["q"], g["sq"], g["k"], g["sk"], g["v"], g["sv"], g["do"], g["sdo"], g["lse"], g["D"], o64,
                      oflip, r["pi"], cu, softmax_scale, docs=docs, kv_heads=kv_heads, shared_stats=True)
    assert np.array_equal(g["pi"], r["pi"]), "pi"
    m = token_mask(cu, T, docs)
    qh = slice(None) if q_heads is None else q_heads
    kh = slice(None) if kv_heads is None else kv_heads
    L1, L2, LA = g["lse"][qh][:, m], lse[qh][:, m], A["lse_a"][qh][:, m]
    lerr = np.abs(L1 - L2)
    say("  stage LSE max|diff| %.3e  max diff/allowance %.3f" % (lerr.max() if lerr.size else 0,
                                                                (lerr / LA).max() if lerr.size else 0))
    assert np.all(lerr <= LA)
    sel = lambda a, hs: a[m][:, hs]
    z = set(zero_in_exact)
    assert_close("O", sel(g["o"], qh), sel(o, qh), sel(oflip, qh), sel(A["o_a"], qh), need_cosine="O" not in z)
    assert_close("dQ", sel(g["dq"], qh), sel(r["dq"], qh), sel(r["dq_flip"], qh), sel(A["dq_a"], qh),
                 need_cosine="dQ" not in z)
    assert_close("dK", sel(g["dk"], kh), sel(r["dk"], kh), sel(r["dk_flip"], kh), sel(A["dk_a"], kh),
                 need_cosine="dK" not in z)
    assert_close("dV", sel(g["dv"], kh), sel(r["dv"], kh), sel(r["dv_flip"], kh), sel(A["dv_a"], kh),
                 need_cosine="dV" not in z)
    return dict(o=o, lse=lse, bwd=r, allow=A)


def bf16_ulp(x):
    """Spacing of BF16 numbers at |x| (subnormal spacing below 2^-126)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def token_mask(cu, T, docs=None):
    m = np.zeros(T, bool)
    cu = np.asarray(cu)
    for i, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        if docs is None or i in docs:
            m[a:b] = True
    return m
