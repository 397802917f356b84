"""Pins for the oracle's replays (CPU only): the forward and backward products computed from
given per-pair decisions (scores, running maxima, E4M3 codes and block exponents).

The GPU parity tests validate each decision the GPU takes against the method's definition and
then compare the GPU's products with these replays on the GPU's own decisions.  Here the
replays are tied to the pinned forward and backward: fed the oracle's own decisions (its
per-pair dumps) they reproduce its outputs bit for bit, on packed ragged documents with several
key tiles, GQA, document offsets and rows outside every document; restricted to a document tail
they reproduce the tail; and a single changed decision moves the output by exactly the change
the method's formula gives (so the replays really read the decisions they are given).

Cited passages: jaehun.me review of FLAMIA, section 1.2 (online softmax, gradient products),
section 3.1 (E4M3 probability operands, dS one scale per 32x32 block, FP16 dQ partial sums),
section 3.2 (dQ prescale)."""
import numpy as np
import pytest

from tests.helpers import bf16_bits
from precision_causal_attention_token_amd import workloads

LOG2E = 1.4426950408889634

CASES = [
    # (T, Hq, Hkv, d, cu)
    (700, 4, 2, 128, [3, 8, 298, 299, 698]),
    (520, 2, 1, 64, [0, 129, 257, 520]),
]


def _setup(orc, case, seed):
    T, Hq, Hkv, d, cu = CASES[case]
    cu = np.array(cu, np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=seed)
    Z = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        Z[name], Z["s" + name] = orc.quantize(bf16_bits(x), cu)
    return T, Hq, Hkv, d, cu, Z, do


def _full_window(T, Hq):
    return dict(row_lo=0, row_hi=T, key_lo=0, key_hi=T, head_lo=0, head_hi=Hq)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_forward_replay_reproduces_oracle(orc, case):
    T, Hq, Hkv, d, cu, Z, _ = _setup(orc, case, 150 + case)
    ss = 1.0 / np.sqrt(d)
    win = _full_window(T, Hq)
    o, lse, o64, dumps = orc.fwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], cu, ss, want_o64=True, window=win)
    r64, rlse = orc.fwd_replay(Z["v"], Z["sv"], cu, win, dumps["fwd_s"], dumps["fwd_m"], dumps["fwd_p"], Hq,
                               ss * LOG2E)
    inside = np.zeros(T, bool)
    for a, b in zip(cu[:-1], cu[1:]):
        inside[a:b] = True
    got = np.transpose(r64, (1, 0, 2))                       # [rows][heads][d]
    assert np.array_equal(got[inside], o64[inside])
    assert np.array_equal(rlse[:, inside].astype(np.float32), lse[:, inside])
    assert np.isnan(got[~inside]).all() and np.isnan(rlse[:, ~inside]).all()
    # every visible pair was dumped, nothing else
    vis = np.zeros((T, T), bool)
    for a, b in zip(cu[:-1], cu[1:]):
        vis[a:b, a:b] = np.tril(np.ones((b - a, b - a), bool))
    assert np.array_equal(~np.isnan(dumps["fwd_s"][0]), vis)


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("causal_dq", [False, True])
def test_backward_replay_reproduces_oracle(orc, case, causal_dq):
    T, Hq, Hkv, d, cu, Z, do = _setup(orc, case, 160 + case)
    ss = 1.0 / np.sqrt(d)
    o, lse, _ = orc.fwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], cu, ss)
    dc, dsc, D = orc.quantize_do(bf16_bits(do), o, cu)
    win = _full_window(T, Hq)
    g = orc.bwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], dc, dsc, lse, D, cu, ss, causal_dq=causal_dq,
                want64=True, window=win)
    w = g["dumps"]
    r = orc.bwd_replay(Z["q"], Z["sq"], Z["k"], Z["sk"], dc, dsc, cu, g["pi"], win, w["bwd_p"], w["bwd_ps"],
                       w["bwd_ds"], w["bwd_dss"], ss)
    inside = np.zeros(T, bool)
    for a, b in zip(cu[:-1], cu[1:]):
        inside[a:b] = True
    assert np.array_equal(np.transpose(r["dq64"], (1, 0, 2))[inside], g["dq64"][inside])
    assert np.array_equal(np.transpose(r["dk64"], (1, 0, 2))[inside], g["dk64"][inside])
    assert np.array_equal(np.transpose(r["dv64"], (1, 0, 2))[inside], g["dv64"][inside])
    # the BF16 outputs follow from the same values
    assert np.array_equal(orc.bf16_rne(np.transpose(r["dq64"], (1, 0, 2))[inside]), g["dq"][inside])


def test_backward_replay_tail_window(orc):
    """A window of the last rows of one document (from a 32-query block of it to its end, all
    keys of the document, one GQA group): dQ of those rows and dK, dV of those keys equal the
    unrestricted backward's."""
    T, Hq, Hkv, d, cu, Z, do = _setup(orc, 1, 170)
    ss = 1.0 / np.sqrt(d)
    o, lse, _ = orc.fwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], cu, ss)
    dc, dsc, D = orc.quantize_do(bf16_bits(do), o, cu)
    a, b = int(cu[2]), int(cu[3])                              # the 263-token document
    win = dict(row_lo=a + 160, row_hi=b, key_lo=a, key_hi=b, head_lo=0, head_hi=Hq)
    full = orc.bwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], dc, dsc, lse, D, cu, ss, want64=True)
    g = orc.bwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], dc, dsc, lse, D, cu, ss, want64=True,
                window=win)
    w = g["dumps"]
    r = orc.bwd_replay(Z["q"], Z["sq"], Z["k"], Z["sk"], dc, dsc, cu, g["pi"], win, w["bwd_p"], w["bwd_ps"],
                       w["bwd_ds"], w["bwd_dss"], ss)
    rows = slice(a + 160, b)
    assert np.array_equal(np.transpose(r["dq64"], (1, 0, 2)), full["dq64"][rows])
    assert np.array_equal(np.transpose(r["dk64"], (1, 0, 2)), full["dk64"][rows])
    assert np.array_equal(np.transpose(r["dv64"], (1, 0, 2)), full["dv64"][rows])


def test_replays_read_the_given_decisions(orc):
    """One changed decision moves the replayed output by exactly the formula's amount:
    forward, one probability code one step up changes O_i by 2^-8 (2^(m_j - m_fin)) delta V_j / l;
    backward, one dShat code one step up changes dK_j by softmax_scale 2^s delta Q_i."""
    T, Hq, Hkv, d, cu, Z, do = _setup(orc, 1, 180)
    ss = 1.0 / np.sqrt(d)
    c = ss * LOG2E
    win = _full_window(T, Hq)
    o, lse, o64, dumps = orc.fwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], cu, ss, want_o64=True, window=win)
    a = int(cu[2])
    h, i, j = 1, 400, a + 20                                  # a row of the third document, key tile 0
    P = dumps["fwd_p"].copy()
    code = int(P[h, i, j])
    assert 0 < code < 0x7E
    P[h, i, j] = code + 1
    base, _ = orc.fwd_replay(Z["v"], Z["sv"], cu, win, dumps["fwd_s"], dumps["fwd_m"], dumps["fwd_p"], Hq, c)
    moved, _ = orc.fwd_replay(Z["v"], Z["sv"], cu, win, dumps["fwd_s"], dumps["fwd_m"], P, Hq, c)
    dec = orc.e4m3_decode(np.array([code, code + 1], np.uint8))
    S, M = dumps["fwd_s"][h, i, a:i + 1], dumps["fwd_m"][h, i, a:i + 1]
    m_fin = M[0]
    l = np.exp2(S * c - m_fin).sum()
    vd = (orc.e4m3_decode(Z["v"][:, 0]) * np.exp2(Z["sv"][0].astype(np.float64) - 127)[:, None])
    expect = 2.0 ** -8 * (dec[1] - dec[0]) * np.exp2(dumps["fwd_m"][h, i, j] - m_fin) * vd[j] / l
    assert np.allclose(moved[h, i] - base[h, i], expect, rtol=1e-9, atol=1e-15)
    others = np.ones(T, bool)
    others[i] = False
    assert np.array_equal(np.nan_to_num(moved[:, others]), np.nan_to_num(base[:, others]))
    # backward: one dShat code
    dc, dsc, D = orc.quantize_do(bf16_bits(do), o, cu)
    g = orc.bwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], dc, dsc, lse, D, cu, ss, window=win)
    w = g["dumps"]
    DS = w["bwd_ds"].copy()
    code = int(DS[h, i, j])
    assert code & 0x7F not in (0, 0x7E, 0x7F)
    DS[h, i, j] = code + 1
    args = (Z["q"], Z["sq"], Z["k"], Z["sk"], dc, dsc, cu, g["pi"], win, w["bwd_p"], w["bwd_ps"])
    r0 = orc.bwd_replay(*args, w["bwd_ds"], w["bwd_dss"], ss)
    r1 = orc.bwd_replay(*args, DS, w["bwd_dss"], ss)
    dec = orc.e4m3_decode(np.array([code, code + 1], np.uint8))
    qd = orc.e4m3_decode(Z["q"][i, h]) * 2.0 ** (int(Z["sq"][h, i]) - 127)
    expect = ss * (dec[1] - dec[0]) * 2.0 ** (int(w["bwd_dss"][h, i, j]) - 127) * qd
    g_kv = h // (Hq // Hkv)
    assert np.allclose(r1["dk64"][g_kv, j] - r0["dk64"][g_kv, j], expect, rtol=1e-9, atol=1e-15)
    assert np.array_equal(np.nan_to_num(r1["dv64"]), np.nan_to_num(r0["dv64"]))
