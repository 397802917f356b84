"""The GPU parity gate itself (CPU only): the stage and chain checks of tests/gpu_common.py run on
a stand-in for a GPU result built from the oracle (its outputs and per-pair decisions, with the
scores stored in FP32 and the running maxima recomputed in FP32 as the kernels define them).
They accept it, and they reject mistakes planted in it: a probability or dShat code one step off
away from any rounding boundary, a block exponent one off, a forward/backward score mismatch, a
dQ partial off by more than the accumulation bound, and a 5e-2 RMS error in one row of O, dQ,
dK or dV."""
import numpy as np
import pytest

from precision_causal_attention_token_amd import workloads
from tests import gpu_common as gc

T, Hq, Hkv, d = 520, 2, 1, 64
CU = np.array([0, 129, 257, 520], np.int32)


def _fake_gpu(orc, causal_dq=False, causal=True):
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=190)
    r = gc.oracle_call(orc, q, k, v, do, CU, causal_dq, causal=causal)
    ss = 1.0 / np.sqrt(d)
    win = gc.full_window(T, Hq)
    _, lse, _, dumps = orc.fwd(r["q"], r["sq"], r["k"], r["sk"], r["v"], r["sv"], CU, ss, want_o64=True, window=win,
                               causal=causal)
    b = orc.bwd(r["q"], r["sq"], r["k"], r["sk"], r["v"], r["sv"], r["do"], r["sdo"], lse, r["D"], CU, ss,
                causal_dq=causal_dq, window=win, causal=causal)
    S = dumps["fwd_s"].astype(np.float32)
    c32 = gc.score_scale32(d)
    M = np.full(S.shape, np.nan, np.float32)
    for a, e in zip(CU[:-1], CU[1:]):
        for i in range(a, e):
            run = np.float32(-np.inf)
            last = i if causal else e - 1
            for kt in range((last - a) // 128, -1, -1):
                cols = slice(a + 128 * kt, min(e, a + 128 * kt + 128, last + 1))
                run = np.maximum(run, (np.nanmax(S[:, i, cols], axis=1) * c32).astype(np.float32))
                M[:, i, cols] = run[:, None]
    g = dict(r)
    g["dumps"] = dict(fwd_s=S, fwd_m=M, fwd_p=dumps["fwd_p"], bwd_s=S.copy(),
                      bwd_dp=b["dumps"]["bwd_dp"].astype(np.float32),
                      **{n: b["dumps"][n] for n in ("bwd_p", "bwd_ps", "bwd_ds", "bwd_dss")})
    g["window"] = win
    g["causal"] = causal
    # each key tile's dQ partial times 2^pi from the oracle's dShat codes, stored in FP32 as the
    # GPU converts it; dQ then follows from those partials as the method forms it
    vis = gc.visible_mask(CU, T, win, causal)
    dsh = orc.e4m3_decode(g["dumps"]["bwd_ds"]) * np.exp2(g["dumps"]["bwd_dss"].astype(np.float64) - 127)
    dsh = np.where(vis[None], dsh, 0.0)
    kd = gc.dequant(r["k"], r["sk"])
    nt = gc.n_key_tiles(win)
    parts = np.full((Hq, T, nt, d), np.nan, np.float32)
    for a, e in zip(CU[:-1], CU[1:]):
        for kt in range(-(-(e - a) // 128)):
            ks = slice(a + 128 * kt, min(e, a + 128 * kt + 128))
            rows = slice(a + 128 * kt if causal else a, e)
            for h in range(Hq):
                parts[h, rows, kt] = (dsh[h, rows, ks] @ kd[ks, h // (Hq // Hkv)]) * \
                    np.exp2(r["pi"][h, rows].astype(np.float64))[:, None]
    g["dumps"]["dq_part"] = parts
    g["dq"] = np.transpose(gc.validate_dq_partials(orc, g, CU, r["pi"], ss), (1, 0, 2)).copy()
    return g, r


def _run(orc, g, r):
    fv = gc.validate_forward(orc, g, CU)
    bv = gc.validate_backward(orc, g, CU)
    gc.chain_check(orc, g, r, CU, fv, bv)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "non-causal"])
def test_gate_accepts_the_oracle_stand_in(orc, causal):
    g, r = _fake_gpu(orc, causal=causal)
    _run(orc, g, r)


def test_gate_rejects_causal_decisions_for_non_causal_attention(orc):
    """The non-causal gate needs the pairs above the diagonal: a causal run fails it."""
    g, r = _fake_gpu(orc)
    g["causal"] = False
    with pytest.raises(AssertionError):
        gc.validate_forward(orc, g, CU)


def _far_from_boundary(orc, codes, values, vis):
    """Index of a visible pair whose value is far from every rounding boundary."""
    dec = orc.e4m3_decode(codes)
    q = np.abs(dec) / 16.0
    far = vis & (np.abs(values - dec) < 0.1 * q) & (np.abs(dec) > 1.0) & ((codes & 0x7F) < 0x7D)
    return tuple(np.argwhere(far)[0])


def test_gate_rejects_a_wrong_probability_code(orc):
    g, r = _fake_gpu(orc)
    du = g["dumps"]
    vis = np.broadcast_to(gc.visible_mask(CU, T, g["window"]), du["fwd_p"].shape)
    c32 = gc.score_scale32(d)
    y = np.exp2(gc.fma32(du["fwd_s"], c32, (np.float32(8) - du["fwd_m"]).astype(np.float32)).astype(np.float64))
    ix = _far_from_boundary(orc, du["fwd_p"], np.where(vis, y, 0), vis)
    du["fwd_p"][ix] += 1
    with pytest.raises(AssertionError, match="probability codes"):
        gc.validate_forward(orc, g, CU)


def test_gate_rejects_a_wrong_dshat_code_and_exponent(orc):
    g, r = _fake_gpu(orc)
    du = g["dumps"]
    vis = np.broadcast_to(gc.visible_mask(CU, T, g["window"]), du["bwd_ds"].shape)
    ix = tuple(np.argwhere(vis & ((du["bwd_ds"] & 0x7F) > 0x40) & ((du["bwd_ds"] & 0x7F) < 0x7D))[7])
    du["bwd_ds"][ix] += 1
    with pytest.raises(AssertionError, match="dShat codes"):
        gc.validate_backward(orc, g, CU)
    g, r = _fake_gpu(orc)
    du = g["dumps"]
    h, i, j = tuple(np.argwhere(du["bwd_ps"] != 0xFF)[100])
    a = int(CU[np.searchsorted(CU, i, side="right") - 1])
    bi, bj = a + 32 * ((i - a) // 32), a + 32 * ((j - a) // 32)
    blk = du["bwd_ps"][h, bi:bi + 32, bj:bj + 32]
    blk[blk != 0xFF] += 1
    with pytest.raises(AssertionError, match="Phat"):
        gc.validate_backward(orc, g, CU)


def test_gate_rejects_a_score_mismatch(orc):
    g, r = _fake_gpu(orc)
    du = g["dumps"]
    ix = tuple(np.argwhere(~np.isnan(du["bwd_s"]))[500])
    du["bwd_s"][ix] = np.nextafter(du["bwd_s"][ix], np.float32(np.inf))
    with pytest.raises(AssertionError):
        gc.validate_forward(orc, g, CU)


@pytest.mark.parametrize("name", ["o", "dq", "dk", "dv"])
def test_gate_rejects_an_error_of_5e2_rms_in_one_row(orc, name):
    g, r = _fake_gpu(orc)
    x = gc.bits_to_f64(g[name])
    scale = gc.rms(x[x != 0])
    row = 300
    x[row, 0, 5] += 5e-2 * scale * np.sign(x[row, 0, 5] or 1.0)
    g[name] = orc.bf16_rne(x)
    with pytest.raises(AssertionError):
        _run(orc, g, r)


def test_gate_rejects_a_wrong_dq_partial(orc):
    g, r = _fake_gpu(orc)
    parts = g["dumps"]["dq_part"]
    ix = tuple(np.argwhere(np.abs(np.nan_to_num(parts)) > 1.0)[3])
    parts[ix] *= np.float32(1.01)
    with pytest.raises(AssertionError, match="dQ partial"):
        gc.validate_backward(orc, g, CU)
