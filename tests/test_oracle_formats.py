"""Pins for the oracle's number formats and token-block quantiser (CPU only).

Cited passages: jaehun.me review of FLAMIA, section 2 (worked example, Fig. 1: E4M3
largest value 448, floor exponent of the OCP conversion), section 3.1 (32 tokens x full
head dim share one power-of-two exponent), section 3.2 (exponents rounded up so nothing
clips), section 3.4 "Packed documents" (statistics never cross a document boundary;
dense per-token scale table); agihunt.info summary (same rules)."""
import json
import os

import numpy as np
import pytest
import torch

from tests.helpers import bf16_bits
from precision_causal_attention_token_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_bf16_f64():
    b = np.arange(65536, dtype=np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def test_e4m3_encoder_matches_torch_cast(orc):
    """Q1: every BF16 pattern times 2^k, k in [-20, 20], against torch's E4M3FN cast (RNE)."""
    x = _all_bf16_f64()
    x = x[np.isfinite(x)]
    ys = np.concatenate([x * 2.0 ** k for k in range(-20, 21)])
    ys = ys[np.isfinite(ys) & (np.abs(ys) <= 464.0)]
    ours = orc.e4m3_rne(ys)
    ref = torch.from_numpy(ys).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert ys.size > 1_000_000
    mism = np.nonzero(ours != ref)[0]
    assert mism.size == 0, (ys[mism[:5]], ours[mism[:5]], ref[mism[:5]])


def test_e4m3_overflow_is_nan_and_decode(orc):
    over = np.array([465.0, 470.0, 1e4, -470.0])
    assert all(c & 0x7F == 0x7F for c in orc.e4m3_rne(over))
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), ~fin)
    assert np.array_equal(ours[fin], ref[fin])
    assert orc.e4m3_decode(np.array([0x7E], np.uint8))[0] == 448.0


def test_e4m3_round_trip_within_half_ulp(orc):
    """Decoded code times 2^s reproduces the element within half a quantum (Q1)."""
    rng = np.random.default_rng(0)
    y = rng.uniform(-448, 448, 200000)
    dec = orc.e4m3_decode(orc.e4m3_rne(y))
    e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
    half_q = 2.0 ** (e - 3) / 2
    assert np.all(np.abs(dec - y) <= half_q * (1 + 1e-12))


def test_e8m0_roundup_definition(orc):
    """Q2: s is the smallest integer with amax <= 448 * 2^s (brute force on the definition)."""
    rng = np.random.default_rng(1)
    a = np.concatenate([np.exp(rng.uniform(-80, 80, 100000)),
                        448.0 * 2.0 ** np.arange(-100, 100),
                        np.nextafter(448.0 * 2.0 ** np.arange(-100, 100), np.inf),
                        2.0 ** np.arange(-120, 120)])
    s = orc.e8m0_roundup(a).astype(np.float64)
    assert np.all(a <= 448.0 * 2.0 ** s)
    free = s > -127                         # minimality holds where the range clamp is inactive
    assert np.all(a[free] > 448.0 * 2.0 ** (s[free] - 1))
    assert np.all(a[~free] <= 448.0 * 2.0 ** -127)
    # boundaries exactly: 448 * 2^k -> k, just above -> k + 1
    k = np.arange(-100, 100)
    assert np.array_equal(orc.e8m0_roundup(448.0 * 2.0 ** k), k)
    assert np.array_equal(orc.e8m0_roundup(np.nextafter(448.0 * 2.0 ** k, np.inf)), k + 1)
    # zero block and range clamp
    assert orc.e8m0_roundup(np.array([0.0]))[0] == -127
    assert orc.e8m0_roundup(np.array([1e-45]))[0] == -127


def test_e8m0_byte_matches_torch_for_powers_of_two(orc):
    k = np.arange(-127, 128)
    s = orc.e8m0_roundup(448.0 * 2.0 ** k)
    ref = torch.from_numpy(2.0 ** k.astype(np.float64)).to(torch.float32).to(torch.float8_e8m0fnu).view(torch.uint8)
    assert np.array_equal((s + 127).astype(np.uint8), ref.numpy())


def test_bf16_rounding_matches_torch_on_float32(orc):
    rng = np.random.default_rng(2)
    with np.errstate(invalid="ignore", over="ignore"):
        x = np.concatenate([rng.standard_normal(100000) * np.exp(rng.uniform(-80, 80, 100000)),
                            (np.arange(1, 1 << 16, dtype=np.uint32) << 15).view(np.float32).astype(np.float64)])
        x = x.astype(np.float32)
    x = x[np.isfinite(x)].astype(np.float64)
    ours = orc.bf16_rne(x)
    ref = bf16_bits(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16))
    assert np.array_equal(ours, ref)


def test_bf16_rounding_near_ties_in_double(orc):
    """Doubles just off a BF16 midpoint (not representable in float32) round the right way."""
    base = np.array([1.0, 3.0, -5.0, 1.5 * 2.0 ** -10, 1.25 * 2.0 ** 70], np.float64)  # even BF16 significands
    e = np.floor(np.log2(np.abs(base)))
    ulp = 2.0 ** (e - 7)
    mid = base + np.sign(base) * ulp / 2          # exact midpoints: tie to even keeps base (even)
    up = mid + np.sign(base) * ulp * 2.0 ** -30
    dn = mid - np.sign(base) * ulp * 2.0 ** -30
    b = orc.bf16_rne(base)
    assert np.array_equal(orc.bf16_rne(mid), b)   # base significands here are even
    assert np.array_equal(orc.bf16_rne(dn), b)
    assert np.array_equal(orc.bf16_rne(up), b + 1)


def test_f16_rounding_matches_numpy(orc):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200000) * np.exp(rng.uniform(-25, 12, 200000)),
                        [65504.0, 65519.9, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26]])
    ours = orc.f16_rne(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def _quant_one_block(orc, values, cu, T, floor_rule):
    x = torch.zeros((T, 1, 1), dtype=torch.bfloat16)
    for t, val in values.items():
        x[t, 0, 0] = val
    return orc.quantize(bf16_bits(x), np.asarray(cu, np.int32), floor_rule=floor_rule)


def test_worked_example_codes_and_scales(orc):
    """Q3: the pages' Fig. 1 at the level of codes and scales (golden fixture)."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))["codes_and_scales"]
    T = 64
    cases = {
        "floor_alone": ({0: 460.0}, [0, T], True),
        "floor_with_future_same_block": ({0: 460.0, 1: 900.0}, [0, T], True),
        "roundup_alone": ({0: 460.0}, [0, T], False),
        "roundup_with_future_same_block": ({0: 460.0, 1: 900.0}, [0, T], False),
        "roundup_with_future_next_block": ({0: 460.0, 32: 900.0}, [0, T], False),
    }
    for name, (vals, cu, fl) in cases.items():
        codes, scales = _quant_one_block(orc, vals, cu, T, fl)
        assert int(scales[0, 0]) == g[name]["scale_byte"], name
        assert int(codes[0, 0, 0]) == g[name]["code"], name
    # the future token in another document leaves the byte and code of 460 unchanged
    codes, scales = _quant_one_block(orc, {0: 460.0, 1: 900.0}, [0, 1, T], T, False)
    assert (int(scales[0, 0]), int(codes[0, 0, 0])) == (128, 118)
    # under the round-up rule no element of the example saturates: decoded |x| <= 448 * 2^s
    codes, scales = _quant_one_block(orc, {0: 460.0, 1: 900.0}, [0, T], T, False)
    dec = orc.e4m3_decode(codes[:2, 0, 0]) * 2.0 ** (scales[0, :2].astype(int) - 127)
    assert np.all(np.abs(dec) <= 448.0 * 2.0)


def test_block_alignment_follows_document_start(orc):
    """R3/Q4: blocks are counted from each document's start, partial last block."""
    T, H, d = 200, 2, 8
    cu = np.array([0, 5, 77, 140, 200], np.int32)
    x = torch.randn((T, H, d), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    big = 5 + 31        # last token of the first block of document 1
    x[big, 0, 3] = 3000.0
    codes, scales = orc.quantize(bf16_bits(x), cu)
    s = scales[0].astype(int)
    assert np.all(s[5:5 + 32] == s[big]) and s[big] >= 127 + 3  # whole doc-aligned block shares it
    assert s[5 + 32] < s[big]                                   # the next block does not
    # within every document, tokens of one 32-block share a byte; blocks never straddle cu
    for a, b in zip(cu[:-1], cu[1:]):
        for t0 in range(a, b, 32):
            t1 = min(t0 + 32, b)
            for h in range(H):
                assert len(set(scales[h, t0:t1].tolist())) == 1


def test_round_up_rule_on_random_blocks(orc):
    """Every block's byte is the smallest non-saturating exponent of its own amax."""
    T, H, d = 300, 3, 16
    cu = np.array([0, 7, 100, 101, 260, 300], np.int32)
    x = (torch.randn((T, H, d), generator=torch.Generator().manual_seed(6)) *
         torch.exp(torch.randn((T, 1, 1), generator=torch.Generator().manual_seed(7)) * 6)).to(torch.bfloat16)
    xf = x.to(torch.float64).numpy()
    codes, scales = orc.quantize(bf16_bits(x), cu)
    for a, b in zip(cu[:-1], cu[1:]):
        for t0 in range(a, b, 32):
            t1 = min(t0 + 32, b)
            for h in range(H):
                amax = np.abs(xf[t0:t1, h]).max()
                s = int(scales[h, t0]) - 127
                assert amax <= 448 * 2.0 ** s and amax > 448 * 2.0 ** (s - 1)
    ref = torch.from_numpy((xf * 2.0 ** -(scales.T[:, :, None].astype(np.float64) - 127)).astype(np.float32))
    assert np.array_equal(codes, ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_document_isolation(orc):
    """Q4 (jaehun.me section 4.7): scaling one document x1e4 leaves every byte of the other
    documents unchanged; a tensor-wide scale would not."""
    lens = workloads.random_lengths(1500, 16, 400, seed=11)
    cu = workloads.cu_seqlens(lens)
    q, k, v, do = workloads.tensors(int(cu[-1]), 4, 4, 64, seed=12)
    c0, s0 = orc.quantize(bf16_bits(k), cu)
    k2 = k.clone()
    a, b = int(cu[2]), int(cu[3])
    k2[a:b] = (k2[a:b].to(torch.float32) * 1e4).to(torch.bfloat16)
    c1, s1 = orc.quantize(bf16_bits(k2), cu)
    other = np.ones(int(cu[-1]), bool)
    other[a:b] = False
    assert np.array_equal(c0[other], c1[other]) and np.array_equal(s0[:, other], s1[:, other])
    assert not np.array_equal(s0[:, a:b], s1[:, a:b])


def test_tokens_outside_documents_are_zero(orc):
    T = 100
    cu = np.array([10, 40, 90], np.int32)
    x = torch.randn((T, 2, 8), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    codes, scales = orc.quantize(bf16_bits(x), cu)
    assert not codes[:10].any() and not codes[90:].any()
    assert not scales[:, :10].any() and not scales[:, 90:].any()


def test_subnormal_block_is_exact(orc):
    """R19: a block of BF16 subnormals is scaled up exactly (no flush)."""
    T = 32
    b = np.zeros((T, 1, 4), np.uint16)
    k = np.arange(T) % 16 + 1
    b[:, 0, 0] = k                            # subnormal BF16 patterns k * 2^-133 (<= 4 significant bits)
    codes, scales = orc.quantize(b, np.array([0, T], np.int32))
    s = int(scales[0, 0]) - 127
    vals = orc.e4m3_decode(codes[:, 0, 0]) * 2.0 ** s
    assert s == -127  # clamp: amax = 16 * 2^-133 would allow s < -127
    assert np.array_equal(vals, k * 2.0 ** -133)
