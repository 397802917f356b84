"""Pins of the oracle's 4-bit score path (jaehun.me §3.1 "Mixed NVFP4/FP8 path", §3.4 "Softmax
throughput"; MXFP4 as the microscaling analogue of the pages' NVFP4): the E2M1 codec, the
round-up exponent of a 32-channel group, the 4-bit copy of Q and K (one exponent per 32 channels
of one token), scores from that copy in the forward and the backward's recomputation, and the
forward's probability operand quantised per 32-key group in the log domain.

Pinned by: the E2M1 values computed from the format's bit fields; rounding properties (every
representable value fixed, midpoints to the even code, nearest everywhere); the exponent rule's
bounds; a hand-worked quantisation; per-token independence; inputs exact in both formats, where
the 4-bit path's scores equal the 8-bit path's and the exact forward and backward agree bit for
bit; one-token documents' closed form; the group exponents' code range; accuracy against exact
attention; the replay reproducing the oracle's own output."""
import numpy as np
import pytest
import torch

import oracle
from precision_causal_attention_token_amd import workloads
from tests.helpers import bf16_bits, bits_to_f64, cosine, exact_attention


def _e2m1_from_fields(c):
    """E2M1 value of a code from its bit fields: sign, 2 exponent bits (bias 1), 1 mantissa bit."""
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    v = m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -v if s else v


def test_e2m1_decode_is_the_format():
    for c in range(16):
        assert oracle.e2m1_decode(c) == _e2m1_from_fields(c), c
    assert sorted({abs(_e2m1_from_fields(c)) for c in range(16)}) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e2m1_rounding():
    vals = np.array([_e2m1_from_fields(c) for c in range(8)])
    # every representable value maps to itself (both signs)
    for c in range(16):
        v = _e2m1_from_fields(c)
        assert oracle.e2m1_decode(oracle.e2m1_rne(v)) == v
    # midpoints go to the code with mantissa bit 0
    for a, b in zip(vals[:-1], vals[1:]):
        mid = 0.5 * (a + b)
        code = int(oracle.e2m1_rne(mid))
        assert code & 1 == 0, (mid, code)
        assert oracle.e2m1_decode(code) in (a, b)
        assert oracle.e2m1_rne(-mid) == code | 8
    # nearest everywhere in range
    rng = np.random.default_rng(5)
    y = rng.uniform(-6, 6, 4000)
    got = np.abs(oracle.e2m1_decode(oracle.e2m1_rne(y)) - y)
    best = np.min(np.abs(np.abs(y)[:, None] - vals[None, :]), axis=1)
    assert np.allclose(got, best, rtol=0, atol=0)
    assert oracle.e2m1_rne(-0.1) == 8                    # sign kept on zero


def test_group_exponent_rounds_up():
    rng = np.random.default_rng(6)
    for a in np.exp2(rng.uniform(-100, 100, 2000)):
        s = oracle.e8m0_roundup4(a)
        assert a <= 6.0 * 2.0 ** s and a > 6.0 * 2.0 ** (s - 1), a
    assert oracle.e8m0_roundup4(0.0) == -127
    assert oracle.e8m0_roundup4(6.0) == 0 and oracle.e8m0_roundup4(6.0000001) == 1


def test_quantiser_hand_example():
    """One token, one head, d = 64: group 0 has amax 6 (exponent 0), group 1 amax 12 (exponent 1)."""
    x = np.zeros((1, 1, 64), np.float32)
    x[0, 0, :4] = [6.0, -3.0, 0.5, 0.3]                  # 0.3 -> 0.5 (nearest)
    x[0, 0, 32:36] = [12.0, 2.9, -1.0, 0.49]              # /2: 6, 1.45 -> 1.5, -0.5, 0.245 -> 0
    xb = torch.from_numpy(x).to(torch.bfloat16)
    codes, scales = oracle.quantize_mx4(bf16_bits(xb), np.array([0, 1], np.int32))
    assert codes.shape == (1, 1, 32) and scales.shape == (1, 1, 2)
    assert list(scales[0, 0]) == [127, 128]
    # two codes per byte, the even channel in the low nibble: 6 = 0x7, -3 = 0xD, 0.5 = 0x1, 0.5 = 0x1
    assert codes[0, 0, 0] == 0xD7 and codes[0, 0, 1] == 0x11
    assert codes[0, 0, 16] == (0x3 << 4) | 0x7 and codes[0, 0, 17] == (0x0 << 4) | 0x9
    assert not codes[0, 0, 2:16].any() and not codes[0, 0, 18:].any()


def test_quantiser_is_per_token_and_bounded():
    T, H, d = 200, 3, 128
    cu = np.array([5, 60, 60, 190], np.int32)
    q, _, _, _ = workloads.tensors(T, H, H, d, seed=1500, outlier_channels=2)
    c, s = oracle.quantize_mx4(bf16_bits(q), cu)
    # outside every document: zero codes and scale bytes
    out = np.r_[0:5, 190:T]
    assert not c[out].any() and not s[:, out].any()
    # each token alone: scrambling the others changes nothing of it
    q2 = q.clone()
    q2[6:] = q2[6:].flip(0) * 8
    c2, s2 = oracle.quantize_mx4(bf16_bits(q2), cu)
    assert np.array_equal(c[5], c2[5]) and np.array_equal(s[:, 5], s2[:, 5])
    # reconstruction: within half the code spacing at the group's exponent (at most 2^s)
    lo = (c & 15).astype(np.int64)
    hi = (c >> 4).astype(np.int64)
    nib = np.stack([lo, hi], -1).reshape(T, H, d)
    dec = np.vectorize(_e2m1_from_fields)(nib) * np.exp2(np.repeat(s.transpose(1, 0, 2), 32, axis=2) - 127.0)
    x = bits_to_f64(bf16_bits(q))
    rows = np.r_[5:190]
    err = np.abs(dec[rows] - x[rows])
    step = np.exp2(np.repeat(s.transpose(1, 0, 2), 32, axis=2)[rows] - 127.0)
    assert (err <= step + 1e-300).all()
    assert (np.abs(dec[rows]) <= 6 * step).all()


def _exact_in_both(T, H, d, seed):
    """BF16 values E2M1 x 2^k with k in [-3, 3] per 32-channel group of each token: exact in the
    4-bit copy, and in the 8-bit token-block copy (a 32-token block's exponent is at least -3)."""
    rng = np.random.default_rng(seed)
    mags = np.array([0.0, 0.5, 1, 1.5, 2, 3, 4, 6])
    v = mags[rng.integers(0, 8, (T, H, d))] * rng.choice([-1.0, 1.0], (T, H, d))
    g = v.reshape(T, H, d // 32, 32)
    g[..., 0] = 6.0                                      # every group's amax is 6 2^k
    k = rng.integers(-3, 4, (T, H, d // 32, 1))
    return torch.from_numpy(g * np.exp2(k)).reshape(T, H, d).to(torch.bfloat16)


def test_scores_from_exact_inputs_match_the_8bit_path():
    """Q, K exact in both formats: the 4-bit path's scores are the 8-bit path's, so with exact
    probabilities the forward's O and LSE, and the exact backward, are bit-identical."""
    T, Hq, Hkv, d = 300, 4, 2, 64
    cu = np.array([0, 140, 141, 300], np.int32)
    q, k = _exact_in_both(T, Hq, d, 1), _exact_in_both(T, Hkv, d, 2)
    _, _, v, do = workloads.tensors(T, Hq, Hkv, d, seed=1501)
    r = {}
    for nm, x in (("q", q), ("k", k), ("v", v)):
        r[nm], r["s" + nm] = oracle.quantize(bf16_bits(x), cu)
    assert np.array_equal(bits_to_f64(bf16_bits(q))[:1], oracle.e4m3_decode(r["q"][:1]) *
                          np.exp2(r["sq"][:, :1].T[:, :, None].astype(np.float64) - 127))
    q4 = oracle.quantize_mx4(bf16_bits(q), cu)
    k4 = oracle.quantize_mx4(bf16_bits(k), cu)
    qk4 = (q4[0], q4[1], k4[0], k4[1])
    args = (r["q"], r["sq"], r["k"], r["sk"], r["v"], r["sv"], cu)
    o8, l8, _ = oracle.fwd(*args, exact_p=True)
    o4, l4, _ = oracle.fwd(*args, exact_p=True, qk4=qk4)
    assert np.array_equal(o8, o4) and np.array_equal(l8.view(np.uint32), l4.view(np.uint32))
    dc, dsc, D = oracle.quantize_do(bf16_bits(do), o8, cu)
    g8 = oracle.bwd(*args[:6], dc, dsc, l8, D, cu, exact=7)
    g4 = oracle.bwd(*args[:6], dc, dsc, l8, D, cu, exact=7, qk4=qk4)
    for nm in ("dq", "dk", "dv"):
        assert np.array_equal(g8[nm], g4[nm]), nm
    # and the 4-bit copy does change the scores of ordinary inputs
    qn, kn, _, _ = workloads.tensors(T, Hq, Hkv, d, seed=1502)
    rq, rsq = oracle.quantize(bf16_bits(qn), cu)
    rk, rsk = oracle.quantize(bf16_bits(kn), cu)
    qn4, kn4 = oracle.quantize_mx4(bf16_bits(qn), cu), oracle.quantize_mx4(bf16_bits(kn), cu)
    a = oracle.fwd(rq, rsq, rk, rsk, r["v"], r["sv"], cu, exact_p=True)[0]
    b = oracle.fwd(rq, rsq, rk, rsk, r["v"], r["sv"], cu, exact_p=True, qk4=(qn4[0], qn4[1], kn4[0], kn4[1]))[0]
    assert not np.array_equal(a, b)


def _chain4(q, k, v, do, cu, window=None):
    r = {}
    for nm, x in (("q", q), ("k", k), ("v", v)):
        r[nm], r["s" + nm] = oracle.quantize(bf16_bits(x), cu)
    q4, k4 = oracle.quantize_mx4(bf16_bits(q), cu), oracle.quantize_mx4(bf16_bits(k), cu)
    qk4 = (q4[0], q4[1], k4[0], k4[1])
    res = oracle.fwd(r["q"], r["sq"], r["k"], r["sk"], r["v"], r["sv"], cu, qk4=qk4, want_o64=True, window=window)
    return r, qk4, res


def test_one_token_documents_closed_form():
    """p = 1: the group exponent is -8 (448 2^-9 < 1 <= 448 2^-8) and the code 256 is exact, so
    O = BF16(deq V)."""
    T, H, d = 40, 2, 64
    cu = np.arange(0, T + 1, dtype=np.int32)
    q, k, v, do = workloads.tensors(T, H, H, d, seed=1503, outlier_channels=2)
    r, qk4, (o, lse, _) = _chain4(q, k, v, do, cu)
    deq = oracle.e4m3_decode(r["v"]) * np.exp2(r["sv"].T[:, :, None].astype(np.float64) - 127)
    assert np.array_equal(o, oracle.bf16_rne(deq))


def test_group_exponents_and_replay():
    """Every (row, tile, 32-key group): one exponent byte, the group's largest code in [224, 448]
    (round-up: no saturation, no wasted exponent step); the replay from the dumps reproduces the
    oracle's O and LSE."""
    T, Hq, Hkv, d = 330, 2, 1, 64
    cu = np.array([0, 330], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=1504, k_dist="student_t3")
    win = dict(row_lo=0, row_hi=T, key_lo=0, key_hi=T, head_lo=0, head_hi=Hq)
    r, qk4, (o, lse, o64, du) = _chain4(q, k, v, do, cu, window=win)
    P, PS, S, M = du["fwd_p"], du["fwd_ps"], du["fwd_s"], du["fwd_m"]
    vis = np.tril(np.ones((T, T), bool))
    n_groups = 0
    for h in range(Hq):
        for i in range(T):
            for g0 in range(0, i + 1, 32):
                g1 = min(g0 + 32, i + 1)
                ps = PS[h, i, g0:g1]
                assert (ps == ps[0]).all()
                vals = oracle.e4m3_decode(P[h, i, g0:g1])
                assert vals.max() <= 448
                if ps[0] > 0:                              # exponent above the clamp
                    assert vals.max() >= 224, (h, i, g0, vals.max())
                n_groups += 1
    assert n_groups > 1000
    c_scale = 1.0 / np.sqrt(d) * 1.4426950408889634
    o_r, l_r = oracle.fwd_replay(r["v"], r["sv"], cu, win, S, M, P, Hq, c_scale, PS=PS)
    assert np.array_equal(np.transpose(o_r, (1, 0, 2)), o64)
    assert np.allclose(l_r, lse.astype(np.float64), rtol=0, atol=1e-5)


def test_log_domain_keeps_small_probabilities():
    """A row whose later 32-key groups hold probabilities near 2^-16 of its maximum, on large
    values: the fixed 2^8 shift rounds them to subnormal or zero codes, the group exponent keeps
    them, and O is closer to the exact-probability output."""
    T, H, d = 128, 1, 64
    cu = np.array([0, T], np.int32)
    rng = np.random.default_rng(7)
    qv = np.zeros((T, H, d)); kv = np.zeros((T, H, d)); vv = rng.standard_normal((T, H, d))
    qv[:, 0, 0] = 1.0
    # keys 32.. score -96 (exact in both copies): 2^(-96 c) = 2^-17.3 of the first group's
    # probabilities, on values 3000 times larger
    kv[:, 0, 0] = np.where(np.arange(T) < 32, 0.0, -96.0)
    vv[32:, 0, :] *= 3000.0
    f = lambda a: torch.from_numpy(a).to(torch.bfloat16)
    q, k, v = f(qv), f(kv), f(vv)
    r = {}
    for nm, x in (("q", q), ("k", k), ("v", v)):
        r[nm], r["s" + nm] = oracle.quantize(bf16_bits(x), cu)
    q4, k4 = oracle.quantize_mx4(bf16_bits(q), cu), oracle.quantize_mx4(bf16_bits(k), cu)
    qk4 = (q4[0], q4[1], k4[0], k4[1])
    args = (r["q"], r["sq"], r["k"], r["sk"], r["v"], r["sv"], cu)
    ex = oracle.fwd(*args, exact_p=True, qk4=qk4, want_o64=True)[2][T - 1]
    log = oracle.fwd(*args, qk4=qk4, want_o64=True)[2][T - 1]
    fixed = oracle.fwd(*args, want_o64=True)[2][T - 1]          # same scores (exact inputs), fixed shift
    e_log, e_fixed = np.abs(log - ex).max(), np.abs(fixed - ex).max()
    assert e_log < 0.25 * e_fixed, (e_log, e_fixed)


def test_four_bit_chain_against_exact_attention():
    """The 4-bit path's O and gradients against exact attention (outlier channels): the coarser
    scores cost accuracy, but the chain stays close (the pages report O cosine 0.9899 for their
    4-bit scores on non-causal inputs)."""
    T, Hq, Hkv, d = 384, 2, 1, 128
    cu = np.array([0, 200, 384], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=1505)
    r, qk4, (o, lse, _) = _chain4(q, k, v, do, cu)
    dc, dsc, D = oracle.quantize_do(bf16_bits(do), o, cu)
    g = oracle.bwd(r["q"], r["sq"], r["k"], r["sk"], r["v"], r["sv"], dc, dsc, lse, D, cu, qk4=qk4)
    f = lambda x: bits_to_f64(bf16_bits(x))
    ref, dq, dk, dv, _ = exact_attention(f(q), f(k), f(v), cu, 1.0 / np.sqrt(d), do=f(do))
    co = cosine(bits_to_f64(o), ref)
    cq = cosine(bits_to_f64(g["dq"]), dq)
    ck = cosine(bits_to_f64(g["dk"]), dk)
    cv = cosine(bits_to_f64(g["dv"]), dv)
    print("4-bit chain vs exact: O %.5f dQ %.5f dK %.5f dV %.5f" % (co, cq, ck, cv))
    assert co > 0.98 and cv > 0.98 and cq > 0.95 and ck > 0.95
