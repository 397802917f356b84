"""Pins for the oracle's forward and backward (CPU only).

Each test ties the oracle to something other than itself: exact FP64 softmax attention
and its autograd gradients (torch, per document), closed forms for special inputs,
invariants of the 32x32 block quantiser, and the causal-leakage probe.

Cited passages: jaehun.me review of FLAMIA, section 1.2 (S = QK^T/sqrt(d), P = softmax(S),
O = PV; dV = P^T dO, dP = dO V^T, dS = P o (dP - D), dQ = dS K, dK = dS^T Q), section 3.1
(probability operands E4M3, dS one scale per 32x32 block, outputs BF16, dQ partials in
FP16), section 3.2 (causal dQ scaling), section 3.3 (D from the quantised dO; dS scale from
the block amax), section 3.4 "Packed documents" (invalid rows get an infinite LSE),
section 4.4 (cosine against an FP32 reference), section 4.5 (leakage probe: perturb
future inputs, compare earlier outputs)."""
import numpy as np
import pytest
import torch

from tests.helpers import bf16_bits, bits_to_f64, cosine, decode_e4m3, dequant, exact_attention
from precision_causal_attention_token_amd import workloads

LOG2E = 1.4426950408889634


def _quantize_all(orc, q, k, v, cu):
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        c, s = orc.quantize(bf16_bits(x), cu)
        out[name], out["s" + name] = c, s
    return out


def _lossless(orc, x, cu):
    """Inputs that are already E4M3 x 2^s per block: quantise-dequantise once (exact in BF16)."""
    c, s = orc.quantize(bf16_bits(x), cu)
    return torch.from_numpy(dequant(c, s)).to(torch.bfloat16)


CASES = [
    # (T, Hq, Hkv, d, cu)
    (300, 2, 2, 64, [0, 300]),
    (700, 4, 2, 128, [3, 8, 298, 299, 698]),
    (520, 2, 1, 64, [0, 129, 257, 520]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_forward_exact_mode_is_softmax_attention(orc, case):
    """A2: with Phat rounding off, the online softmax over descending key tiles equals FP64
    softmax attention on the decoded operands; rows outside documents get O = 0, LSE = inf."""
    T, Hq, Hkv, d, cu = CASES[case]
    cu = np.array(cu, np.int32)
    q, k, v, _ = workloads.tensors(T, Hq, Hkv, d, seed=40 + case)
    Qz = _quantize_all(orc, q, k, v, cu)
    ss = 1.0 / np.sqrt(d)
    o, lse, o64 = orc.fwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], cu, ss, exact_p=True, want_o64=True)
    qd, kd, vd = dequant(Qz["q"], Qz["sq"]), dequant(Qz["k"], Qz["sk"]), dequant(Qz["v"], Qz["sv"])
    ref = exact_attention(qd, kd, vd, cu, ss)
    assert np.abs(o64 - ref).max() <= 1e-12 * np.abs(ref).max()
    # LSE in log2 units against log-sum-exp of the exact scores
    grp = Hq // Hkv
    for a, b in zip(cu[:-1], cu[1:]):
        for h in range(Hq):
            S = ss * qd[a:b, h] @ kd[a:b, h // grp].T
            S[np.triu_indices(b - a, 1)] = -np.inf
            mx = S.max(1)
            ref_lse = (mx + np.log(np.exp(S - mx[:, None]).sum(1))) * LOG2E
            assert np.allclose(lse[h, a:b], ref_lse, rtol=2e-7, atol=1e-6)
    outside = np.ones(T, bool)
    for a, b in zip(cu[:-1], cu[1:]):
        outside[a:b] = False
    assert np.all(np.isinf(lse[:, outside])) and not o[outside].any()


def test_forward_probability_rounding_closed_form(orc):
    """Two keys: O_1 = (Phat_0 V_0 + Phat_1 V_1) / (p_0 + p_1) with Phat = E4M3(2^8 p)/2^8
    (torch's cast), l summed from the unrounded p; and the rounding is really applied."""
    T, d = 2, 64
    q = torch.zeros((T, 1, d)); k = torch.zeros((T, 1, d)); v = torch.zeros((T, 1, d))
    q[1, 0, 0] = 3.0
    k[0, 0, 0] = 1.75; k[1, 0, 0] = 0.8125
    v[0, 0, :] = torch.linspace(-2, 2, d); v[1, 0, :] = 1.5
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    cu = np.array([0, 2], np.int32)
    Qz = _quantize_all(orc, q, k, v, cu)
    ss = 0.7
    _, lse, o64 = orc.fwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], cu, ss, want_o64=True)
    qd, kd, vd = dequant(Qz["q"], Qz["sq"]), dequant(Qz["k"], Qz["sk"]), dequant(Qz["v"], Qz["sv"])
    t = ss * LOG2E * (kd[:, 0] @ qd[1, 0])
    p = np.exp2(t - t.max())
    ph = torch.from_numpy(p * 256).to(torch.float8_e4m3fn).to(torch.float64).numpy() / 256
    assert not np.allclose(ph, p)  # this input exercises the rounding
    expect = (ph[0] * vd[0, 0] + ph[1] * vd[1, 0]) / p.sum()
    assert np.abs(o64[1, 0] - expect).max() <= 1e-14
    assert np.isclose(lse[0, 1], t.max() + np.log2(p.sum()), rtol=1e-7)


def test_forward_accuracy_against_exact_fp32_inputs(orc):
    """A1 (spec yardstick): O cosine >= 0.998 against exact attention on the
    unquantised BF16 inputs (one 256-token document, 2 heads, d = 64)."""
    cu, shp, (q, k, v, do) = workloads.workload("single")
    Qz = _quantize_all(orc, q, k, v, cu)
    ss = 1.0 / np.sqrt(shp.d)
    o, lse, o64 = orc.fwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], cu, ss, want_o64=True)
    f = lambda x: x.to(torch.float64).numpy()
    ref, dq, dk, dv, _ = exact_attention(f(q), f(k), f(v), cu, ss, do=f(do))
    assert cosine(bits_to_f64(o), ref) >= 0.998
    dc, ds_, D = orc.quantize_do(bf16_bits(do), o, cu)
    g = orc.bwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], dc, ds_, lse, D, cu, ss)
    cos = [cosine(bits_to_f64(g[n]), r) for n, r in (("dq", dq), ("dk", dk), ("dv", dv))]
    assert min(cos) >= 0.99, cos


@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_exact_mode_is_autograd(orc, case):
    """With the P, dS and FP16 roundings off, the backward equals FP64 autograd of softmax
    attention on the decoded operands (dQ, dK incl. the softmax scale; GQA group sums)."""
    T, Hq, Hkv, d, cu = CASES[case]
    cu = np.array(cu, np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=60 + case)
    Qz = _quantize_all(orc, q, k, v, cu)
    ss = 1.0 / np.sqrt(d)
    _, lse, o64 = orc.fwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], cu, ss, exact_p=True, want_o64=True)
    dc, dsc = orc.quantize(bf16_bits(do), cu)
    dod = dequant(dc, dsc)
    D = np.einsum("thc,thc->ht", dod, o64).astype(np.float32)
    g = orc.bwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], dc, dsc, lse, D, cu, ss,
                causal_dq=True, exact=7, want64=True)
    qd, kd, vd = dequant(Qz["q"], Qz["sq"]), dequant(Qz["k"], Qz["sk"]), dequant(Qz["v"], Qz["sv"])
    _, rq, rk, rv, _ = exact_attention(qd, kd, vd, cu, ss, do=dod)
    for name, ref in (("dq64", rq), ("dk64", rk), ("dv64", rv)):
        assert np.abs(g[name] - ref).max() <= 2e-6 * np.abs(ref).max(), name


def test_backward_block_quantisers(orc):
    """The P and dS operands of the gradient products: per 32x32 document-aligned block, the
    exponent is the round-up exponent of the block amax (so the largest code magnitude lies
    in [224, 448]), and the codes approximate the exact softmax P and dS = dL/dS (autograd)
    to E4M3 precision."""
    T, H, d = 200, 2, 64
    cu = np.array([0, T], np.int32)
    q, k, v, do = workloads.tensors(T, H, H, d, seed=71)
    Qz = _quantize_all(orc, q, k, v, cu)
    ss = 1.0 / np.sqrt(d)
    # exact forward statistics, so that P and dS below are those of exact attention
    _, lse, o64 = orc.fwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], cu, ss, exact_p=True, want_o64=True)
    dc, dsc = orc.quantize(bf16_bits(do), cu)
    dod = dequant(dc, dsc)
    D = np.einsum("thc,thc->ht", dod, o64).astype(np.float32)
    g = orc.bwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], dc, dsc, lse, D, cu, ss, debug=True)
    qd, kd, vd = dequant(Qz["q"], Qz["sq"]), dequant(Qz["k"], Qz["sk"]), dequant(Qz["v"], Qz["sv"])
    # exact P from the stored LSE, and dS as the gradient of the score with D from the stored O
    nb = (T + 31) // 32
    for h in range(H):
        S = ss * qd[:, h] @ kd[:, h].T
        mask = np.tril(np.ones((T, T), bool))
        P = np.where(mask, np.exp2(S * LOG2E - lse[h][:, None].astype(np.float64)), 0.0)
        dP = dod[:, h] @ vd[:, h].T
        dS = P * (dP - D[h][:, None].astype(np.float64))
        # autograd cross-check of dS on the exact forward (independent of the oracle's formula)
        St = torch.tensor(S, requires_grad=True)
        Pt = torch.softmax(St.masked_fill(~torch.from_numpy(mask), float("-inf")), -1)
        Ot = Pt @ torch.from_numpy(vd[:, h])
        Ot.backward(torch.from_numpy(dod[:, h]))
        assert np.abs(St.grad.numpy() - dS).max() <= 1e-5 * np.abs(dS).max()
        for bq in range(nb):
            for bk in range(bq + 1):
                rs, cs = slice(32 * bq, min(32 * bq + 32, T)), slice(32 * bk, min(32 * bk + 32, T))
                for ref, sc, code in ((P, g["p_scale"], g["p_code"]), (dS, g["ds_scale"], g["ds_code"])):
                    s = int(sc[h, bq, bk]) - 127
                    dec = decode_e4m3(code[h, rs, cs])
                    if np.abs(ref[rs, cs]).max() == 0:
                        assert s == -127 and not dec.any()
                        continue
                    assert 224 <= np.abs(dec).max() <= 448
                    err = np.abs(dec * 2.0 ** s - ref[rs, cs])
                    assert np.all(err <= 2.0 ** -4 * np.abs(ref[rs, cs]) + 2.0 ** (s - 10) * 1.0001)


def test_query_zero_closed_form(orc):
    """A3: Q = 0 gives t = 0, p = 1, Phat = 256 exactly: O_i is the running mean of the decoded
    V rows, LSE_i = log2(i + 1), and dV_j = sum_{i >= j} deq(dO_i) / (i + 1) up to the E4M3
    rounding of the P blocks."""
    T, H, d = 300, 1, 64
    cu = np.array([0, T], np.int32)
    _, k, v, do = workloads.tensors(T, H, H, d, seed=81)
    q = torch.zeros((T, H, d), dtype=torch.bfloat16)
    Qz = _quantize_all(orc, q, k, v, cu)
    ss = 1.0 / np.sqrt(d)
    o, lse, o64 = orc.fwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], cu, ss, want_o64=True)
    vd = dequant(Qz["v"], Qz["sv"])[:, 0]
    n = np.arange(1, T + 1)[:, None]
    assert np.abs(o64[:, 0] - np.cumsum(vd, 0) / n).max() <= 1e-13
    assert np.array_equal(lse[0], np.log2(np.arange(1, T + 1)).astype(np.float32))
    dc, dsc, D = orc.quantize_do(bf16_bits(do), o, cu)
    g = orc.bwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], dc, dsc, lse, D, cu, ss, want64=True)
    dod = dequant(dc, dsc)[:, 0]
    W = np.tril(np.ones((T, T))) / n              # P_ij = 1/(i+1) for j <= i
    ref = W.T @ dod
    bound = 2.0 ** -4 * (np.abs(W).T @ np.abs(dod)) + 1e-12
    assert np.all(np.abs(g["dv64"][:, 0] - ref) <= bound)


def test_one_token_documents(orc):
    """A4: every document is a single token: O = BF16(deq V), dV = BF16(deq dO) bit-exactly
    (as sums from +0: an E4M3 negative zero gives +0), LSE = t_ii.  dS = P (dP - D) vanishes up
    to the FP32 storage of LSE and D (P = 1 and D = dP in exact arithmetic), so dQ and dK are
    at rounding level."""
    T, H, d = 96, 2, 128
    cu = workloads.cu_seqlens([1] * T)
    q, k, v, do = workloads.tensors(T, H, H, d, seed=91)
    Qz = _quantize_all(orc, q, k, v, cu)
    ss = 1.0 / np.sqrt(d)
    o, lse, _ = orc.fwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], cu, ss)
    vd = dequant(Qz["v"], Qz["sv"]) + 0.0
    assert np.array_equal(o, bf16_bits(torch.from_numpy(vd).to(torch.bfloat16)))
    qd, kd = dequant(Qz["q"], Qz["sq"]), dequant(Qz["k"], Qz["sk"])
    t = (qd * kd).sum(-1).T * ss * LOG2E
    assert np.allclose(lse, t, rtol=1e-6, atol=1e-6)
    dc, dsc, D = orc.quantize_do(bf16_bits(do), o, cu)
    g = orc.bwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], dc, dsc, lse, D, cu, ss)
    assert np.array_equal(g["dv"], bf16_bits(torch.from_numpy(dequant(dc, dsc) + 0.0).to(torch.bfloat16)))
    dv_max = np.abs(bits_to_f64(g["dv"])).max()
    assert np.abs(bits_to_f64(g["dq"])).max() <= 1e-5 * dv_max
    assert np.abs(bits_to_f64(g["dk"])).max() <= 1e-5 * dv_max


def test_d_identity_on_lossless_inputs(orc):
    """A5 (jaehun.me section 3.3): D_i = dO_i . O_i equals sum_j P_ij dP_ij up to the output's
    rounding, and each row of dS sums to ~0."""
    T, H, d = 256, 2, 64
    cu = np.array([0, 100, T], np.int32)
    q, k, v, do = workloads.tensors(T, H, H, d, seed=101)
    q, k, v = (_lossless(orc, x, cu) for x in (q, k, v))
    Qz = _quantize_all(orc, q, k, v, cu)
    ss = 1.0 / np.sqrt(d)
    o, lse, _ = orc.fwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], cu, ss, exact_p=True)
    dc, dsc, D = orc.quantize_do(bf16_bits(do), o, cu)
    qd, kd, vd, dod = (dequant(Qz["q"], Qz["sq"]), dequant(Qz["k"], Qz["sk"]), dequant(Qz["v"], Qz["sv"]),
                       dequant(dc, dsc))
    for a, b in zip(cu[:-1], cu[1:]):
        for h in range(H):
            S = ss * qd[a:b, h] @ kd[a:b, h].T
            S[np.triu_indices(b - a, 1)] = -np.inf
            P = np.exp(S - S.max(1, keepdims=True)); P /= P.sum(1, keepdims=True)
            dP = dod[a:b, h] @ vd[a:b, h].T
            ref = (P * dP).sum(1)
            assert np.abs(D[h, a:b] - ref).max() <= 1e-2 * np.abs(ref).max()
            dS = P * (dP - D[h, a:b][:, None])
            assert np.abs(dS.sum(1)).max() <= 1e-2 * np.abs(dS).max() * 10


def test_gqa_equals_duplicated_heads(orc):
    """A6: a GQA call equals the MHA call with K/V heads duplicated; its dK/dV are the sums
    over each group's query heads."""
    T, Hq, Hkv, d = 300, 4, 2, 64
    cu = np.array([0, 140, T], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=111)
    ss = 1.0 / np.sqrt(d)
    res = []
    for kk, vv in ((k, v), (k.repeat_interleave(2, 1), v.repeat_interleave(2, 1))):
        Qz = _quantize_all(orc, q, kk, vv, cu)
        o, lse, _ = orc.fwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], cu, ss)
        dc, dsc, D = orc.quantize_do(bf16_bits(do), o, cu)
        g = orc.bwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], dc, dsc, lse, D, cu, ss,
                    causal_dq=True, want64=True)
        res.append((o, lse, g))
    (o1, l1, g1), (o2, l2, g2) = res
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and np.array_equal(g1["dq"], g2["dq"])
    for name in ("dk64", "dv64"):
        summed = g2[name].reshape(T, Hkv, 2, d).sum(2)
        assert np.abs(g1[name] - summed).max() <= 1e-12 * np.abs(summed).max()


def _perturb(x, a, b0, b, scale):
    y = x.clone()
    y[a + b0:b] = (y[a + b0:b].to(torch.float32) * scale).to(torch.bfloat16)
    return y


@pytest.mark.parametrize("b0", [32, 160])
def test_leakage_probe(orc, b0):
    """L1/L2 (jaehun.me section 4.5): perturbing Q, K, V at every token of a document from
    offset b0 (a block boundary) on leaves O, LSE of earlier rows and of the other documents
    bit-identical; with the causal dQ scale and dO zeroed on the perturbed suffix, dQ, dK,
    dV there are bit-identical too.  With the sequence-wide dQ scale the exponent pi of
    earlier rows moves (the documented residual dependence, jaehun.me section 3.2)."""
    T, Hq, Hkv, d = 520, 4, 2, 64
    cu = np.array([0, 300, T], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=121)
    a, b = 0, 300
    do = do.clone()
    do[a + b0:b] = 0
    ss = 1.0 / np.sqrt(d)
    keep = np.ones(T, bool)
    keep[a + b0:b] = False
    runs = []
    for scale in (1.0, 1024.0):
        qq, kk, vv = (_perturb(x, a, b0, b, scale) for x in (q, k, v))
        Qz = _quantize_all(orc, qq, kk, vv, cu)
        o, lse, _ = orc.fwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], cu, ss)
        dc, dsc, D = orc.quantize_do(bf16_bits(do), o, cu)
        gc = orc.bwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], dc, dsc, lse, D, cu, ss, causal_dq=True)
        gd = orc.bwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], dc, dsc, lse, D, cu, ss, causal_dq=False)
        runs.append((o, lse, gc, gd))
    (o0, l0, c0, d0), (o1, l1, c1, d1) = runs
    assert not np.array_equal(o0, o1)                          # the perturbation did something
    assert np.array_equal(o0[keep], o1[keep]) and np.array_equal(l0[:, keep], l1[:, keep])
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(c0[n][keep], c1[n][keep]), n
    assert np.array_equal(c0["pi"][:, keep], c1["pi"][:, keep])
    assert not np.array_equal(d0["pi"][:, keep], d1["pi"][:, keep])


@pytest.mark.parametrize("causal_dq", [False, True])
def test_backward_tail_restriction_is_exact(orc, causal_dq):
    """The oracle's tail_blocks work restriction (used to sample long documents on the GPU)
    visits only the last query blocks of each document: dQ of those rows and dK, dV of the
    keys in those blocks equal the unrestricted backward bit for bit (ragged documents, a
    partial last block, GQA, several key tiles)."""
    T, Hq, Hkv, d = 900, 4, 2, 64
    cu = np.array([0, 611, 640, 900], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=123)
    Qz = _quantize_all(orc, q, k, v, cu)
    o, lse, _ = orc.fwd(Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], cu)
    dc, dsc, D = orc.quantize_do(bf16_bits(do), o, cu)
    args = (Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], dc, dsc, lse, D, cu)
    full = orc.bwd(*args, causal_dq=causal_dq, want64=True)
    tail_blocks = 5
    part = orc.bwd(*args, causal_dq=causal_dq, want64=True, tail_blocks=tail_blocks)
    assert np.array_equal(full["pi"], part["pi"])
    covered = 0
    for a, b in zip(cu[:-1], cu[1:]):
        L = b - a
        nb = (L + 31) // 32
        t0 = a + 32 * max(nb - tail_blocks, 0)   # first row / key of the complete tail
        for name in ("dq", "dk", "dv", "dq64", "dk64", "dv64"):
            assert np.array_equal(full[name][t0:b], part[name][t0:b]), (name, a, b)
        covered += b - t0
        if t0 > a:  # earlier keys hold partial sums: the restriction really skipped work
            assert not np.array_equal(full["dk64"][a:t0], part["dk64"][a:t0])
    assert covered < T


def test_forward_tail_restriction_is_exact(orc):
    """The oracle's tail_rows work restriction (used to sample long documents on the GPU)
    computes the last rows of each document exactly as the unrestricted forward does."""
    T, Hq, Hkv, d = 900, 4, 2, 64
    cu = np.array([0, 611, 640, 900], np.int32)
    q, k, v, _ = workloads.tensors(T, Hq, Hkv, d, seed=124)
    Qz = _quantize_all(orc, q, k, v, cu)
    args = (Qz["q"], Qz["sq"], Qz["k"], Qz["sk"], Qz["v"], Qz["sv"], cu)
    o, lse, o64 = orc.fwd(*args, want_o64=True)
    tail = 70
    o2, lse2, o642 = orc.fwd(*args, want_o64=True, tail_rows=tail)
    for a, b in zip(cu[:-1], cu[1:]):
        t0 = max(a, b - tail)
        assert np.array_equal(o[t0:b], o2[t0:b]) and np.array_equal(o64[t0:b], o642[t0:b])
        assert np.array_equal(lse[:, t0:b], lse2[:, t0:b])
        if t0 > a:  # earlier rows were skipped
            assert np.all(np.isnan(lse2[:, a:t0]))
