"""Pins for the oracle's non-causal variant (CPU only): every key of a row's document is
visible; the forward visits the document's key tiles from the last one down to tile 0, the
running maximum updated once per tile.  Batched calls are documents of equal length.

Pinned against exact FP64 softmax attention without the causal mask (autograd for the
gradients), closed forms (Q = 0: every row is the mean of its document's V; the last row of a
document sees the same keys in the same tile order as the causal forward), the replays, and
brute force for the non-causal work lists.

Cited passages: jaehun.me review of FLAMIA, section 1.2 (attention forward and backward),
section 3.4 "Work scheduling" (a static serpentine schedule for non-causal calls; every item of
a document then visits the same key blocks), section 5.1 (non-causal paths named as the
variant beside the causal one)."""
import numpy as np
import pytest
import torch

from tests.helpers import bf16_bits, dequant, exact_attention
from precision_causal_attention_token_amd import workloads

LOG2E = 1.4426950408889634

CASES = [
    # (T, Hq, Hkv, d, cu)
    (700, 4, 2, 128, [3, 8, 298, 299, 698]),
    (520, 2, 1, 64, [0, 129, 257, 520]),
    (512, 2, 2, 64, [0, 128, 256, 384, 512]),   # batched: four sequences of 128
]


def _quantize_all(orc, q, k, v, cu):
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        out[name], out["s" + name] = orc.quantize(bf16_bits(x), cu)
    return out


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noncausal_exact_modes_are_attention(orc, case):
    T, Hq, Hkv, d, cu = CASES[case]
    cu = np.array(cu, np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=210 + case)
    Z = _quantize_all(orc, q, k, v, cu)
    ss = 1.0 / np.sqrt(d)
    o, lse, o64 = orc.fwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], cu, ss, exact_p=True, want_o64=True,
                          causal=False)
    qd, kd, vd = dequant(Z["q"], Z["sq"]), dequant(Z["k"], Z["sk"]), dequant(Z["v"], Z["sv"])
    dc, dsc = orc.quantize(bf16_bits(do), cu)
    dod = dequant(dc, dsc)
    ref, rq, rk, rv, _ = exact_attention(qd, kd, vd, cu, ss, do=dod, causal=False)
    assert np.abs(o64 - ref).max() <= 1e-12 * np.abs(ref).max()
    grp = Hq // Hkv
    for a, b in zip(cu[:-1], cu[1:]):
        for h in range(Hq):
            S = ss * qd[a:b, h] @ kd[a:b, h // grp].T
            mx = S.max(1)
            assert np.allclose(lse[h, a:b], (mx + np.log(np.exp(S - mx[:, None]).sum(1))) * LOG2E, rtol=2e-7, atol=1e-6)
    outside = np.ones(T, bool)
    for a, b in zip(cu[:-1], cu[1:]):
        outside[a:b] = False
    assert np.all(np.isinf(lse[:, outside])) and not o[outside].any()
    D = np.einsum("thc,thc->ht", dod, o64).astype(np.float32)
    g = orc.bwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], dc, dsc, lse, D, cu, ss, exact=7, want64=True,
                causal=False)
    for name, r in (("dq64", rq), ("dk64", rk), ("dv64", rv)):
        assert np.abs(g[name] - r).max() <= 2e-6 * np.abs(r).max(), name
    # the causal variant differs (the mask matters on these inputs)
    oc, _, _ = orc.fwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], cu, ss, exact_p=True)
    assert not np.array_equal(oc, o)


def test_noncausal_closed_forms(orc):
    """Q = 0: t = 0 everywhere, every probability is 1 (code 256 exactly), so O_i is the mean of
    the document's decoded V rows.  The last row of each document sees the same keys, in the same
    tile order, as in the causal forward: bit-identical O and LSE there."""
    T, H, d = 600, 1, 64
    cu = np.array([0, 300, 600], np.int32)
    _, k, v, _ = workloads.tensors(T, H, H, d, seed=220)
    q = torch.zeros((T, H, d), dtype=torch.bfloat16)
    Z = _quantize_all(orc, q, k, v, cu)
    o, lse, o64 = orc.fwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], cu, want_o64=True, causal=False)
    vd = dequant(Z["v"], Z["sv"])[:, 0]
    for a, b in zip(cu[:-1], cu[1:]):
        assert np.abs(o64[a:b, 0] - vd[a:b].mean(0)).max() <= 1e-13
        assert np.all(lse[0, a:b] == np.float32(np.log2(b - a)))
    q, k, v, _ = workloads.tensors(T, 2, 2, d, seed=221)
    Z = _quantize_all(orc, q, k, v, cu)
    args = (Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], cu)
    on, ln, _ = orc.fwd(*args, causal=False)
    oc, lc, _ = orc.fwd(*args)
    last = cu[1:] - 1
    assert np.array_equal(on[last], oc[last]) and np.array_equal(ln[:, last], lc[:, last])
    assert not np.array_equal(on[last - 1], oc[last - 1])


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noncausal_replays_reproduce_oracle(orc, case):
    T, Hq, Hkv, d, cu = CASES[case]
    cu = np.array(cu, np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=230 + case)
    Z = _quantize_all(orc, q, k, v, cu)
    ss = 1.0 / np.sqrt(d)
    win = dict(row_lo=0, row_hi=T, key_lo=0, key_hi=T, head_lo=0, head_hi=Hq)
    o, lse, o64, du = orc.fwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], cu, ss, want_o64=True, window=win,
                              causal=False)
    r64, rlse = orc.fwd_replay(Z["v"], Z["sv"], cu, win, du["fwd_s"], du["fwd_m"], du["fwd_p"], Hq, ss * LOG2E,
                               causal=False)
    inside = np.zeros(T, bool)
    for a, b in zip(cu[:-1], cu[1:]):
        inside[a:b] = True
    assert np.array_equal(np.transpose(r64, (1, 0, 2))[inside], o64[inside])
    dc, dsc, D = orc.quantize_do(bf16_bits(do), o, cu)
    g = orc.bwd(Z["q"], Z["sq"], Z["k"], Z["sk"], Z["v"], Z["sv"], dc, dsc, lse, D, cu, ss, want64=True,
                window=win, causal=False)
    w = g["dumps"]
    r = orc.bwd_replay(Z["q"], Z["sq"], Z["k"], Z["sk"], dc, dsc, cu, g["pi"], win, w["bwd_p"], w["bwd_ps"],
                       w["bwd_ds"], w["bwd_dss"], ss, causal=False)
    for nm in ("dq64", "dk64", "dv64"):
        assert np.array_equal(np.transpose(r[nm], (1, 0, 2))[inside], g[nm][inside]), nm
    # every pair of a document was visited, above the diagonal too
    vis = np.zeros((T, T), bool)
    for a, b in zip(cu[:-1], cu[1:]):
        vis[a:b, a:b] = True
    assert np.array_equal(~np.isnan(du["fwd_s"][0]), vis)


@pytest.mark.parametrize("kind", [2, 3])
def test_noncausal_worklists_brute_force(orc, kind):
    rng = np.random.default_rng(240 + kind)
    for trial in range(30):
        lens = rng.integers(0, 700, rng.integers(1, 12))
        cu = workloads.cu_seqlens(lens.tolist())
        G = int(rng.integers(1, 9))
        got = orc.worklist(cu, kind, G)
        ref = []
        for k, L in enumerate(lens):
            nb = (L + 255) // 256 if kind == 2 else (L + 127) // 128
            # equal costs: documents of more than 8 tokens first (short ones close the list)
            ref += [(-((L + 127) // 128), int(L <= 8), k, b) for b in range(nb)]
        ref.sort()
        assert len(got) == len(ref)
        for i, ((negc, _, k, b), row) in enumerate(zip(ref, got)):
            r, w = divmod(i, G)
            assert tuple(row) == (k, b, -negc, w if r % 2 == 0 else G - 1 - w)
