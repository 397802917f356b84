"""GPU parity of the 4-bit score path (jaehun.me §3.1 "Mixed NVFP4/FP8 path", §3.4 "Softmax
throughput"; MXFP4 as the microscaling analogue of the pages' NVFP4) against the oracle, through
the C ABI: the quantiser's 4-bit copy of Q and K bit-exact (and the 8-bit codes unchanged beside
it); then, per case, the stage checks (forward scores from the 4-bit copies bit-identical to the
backward's recomputation and within the accumulation bound of the 4-bit codes' exact dot
products, running maxima, every 32-key group exponent and probability code of the log-domain
operand, every backward decision, products against the oracle's replays at 2e-2 RMS + 1 BF16
ulp) and the chain against the oracle's own 4-bit chain."""
import numpy as np
import pytest
import torch

import precision_causal_attention_token_amd as fl
from precision_causal_attention_token_amd import workloads
from tests import gpu_common as gc
from tests.helpers import bf16_bits, bits_to_f64, cosine, exact_attention

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,rot", [(64, False), (128, False), (128, True)])
def test_mx4_quantiser_bit_exact(orc, d, rot):
    T, Hq, Hkv = 1200, 4, 2
    cu = np.array([9, 40, 41, 555, 555, 1100], np.int32)
    q, k, v, _ = workloads.tensors(T, Hq, Hkv, d, seed=1600 + d + rot, outlier_channels=2)
    cu_d = torch.as_tensor(cu).cuda()
    out = fl.quantize([q.cuda(), k.cuda(), v.cuda()], cu_d, hadamard=(rot, rot, False), mx4=(True, True, False))
    torch.cuda.synchronize()
    assert len(out[2]) == 2
    for x, o in ((q, out[0]), (k, out[1])):
        rc, rs = orc.quantize_mx4(bf16_bits(x), cu, hadamard=rot)
        assert np.array_equal(o[2].cpu().numpy(), rc) and np.array_equal(o[3].cpu().numpy(), rs)
        c8, s8 = orc.quantize(bf16_bits(x), cu, hadamard=rot)
        assert np.array_equal(o[0].cpu().numpy(), c8) and np.array_equal(o[1].cpu().numpy(), s8)
    gc.say("  4-bit copy d=%d rotated=%s: codes and exponents bit-exact, 8-bit codes unchanged" % (d, rot))


def test_mx4_quantiser_full_size(orc):
    """The 65536-token workload's Q and K (16 heads, d = 128, Student-t K)."""
    cu, shp, (q, k, v, do) = workloads.workload("long")
    cu_d = torch.as_tensor(cu).cuda()
    out = fl.quantize([q.cuda(), k.cuda()], cu_d, mx4=True)
    torch.cuda.synchronize()
    for x, o in ((q, out[0]), (k, out[1])):
        rc, rs = orc.quantize_mx4(bf16_bits(x), cu)
        assert np.array_equal(o[2].cpu().numpy(), rc) and np.array_equal(o[3].cpu().numpy(), rs)
    gc.say("  4-bit copy of the 65536-token workload's Q and K: bit-exact")


CASES = [
    ("packed-d128-outliers", 1100, 4, 2, 128, [0, 300, 301, 700, 1100], dict(outlier_channels=2), True),
    ("offsets-gqa4-d64-empty", 1200, 4, 1, 64, [9, 40, 41, 555, 555, 1100], {}, True),
    ("ragged-d128-studentt", 1000, 2, 2, 128, [0, 129, 383, 385, 1000], dict(k_dist="student_t3"), True),
    ("one-4096-d128-8wave", 4096, 2, 2, 128, [0, 4096], {}, True),
    ("noncausal-d128", 1000, 2, 2, 128, [0, 400, 401, 1000], dict(outlier_channels=2), False),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_mx4_parity(orc, case):
    name, T, Hq, Hkv, d, cu, opts, causal = CASES[case]
    gc.say("4-bit scores %s" % name)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=1610 + case, **opts)
    cu = np.asarray(cu, np.int32)
    gc.stage_and_chain(orc, q, k, v, do, cu, gc.full_window(T, Hq), causal=causal, qk4=True)


def test_mx4_with_rotation(orc):
    """4-bit copies of rotated Q and K (the rotation inside the quantiser, before both copies):
    stage and chain against the oracle's rotated 4-bit chain (dQ, dK compared in the rotated
    basis, as the other rotation tests do)."""
    T, Hq, Hkv, d = 1100, 4, 2, 128
    cu = np.array([0, 300, 301, 700, 1100], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=1640, outlier_channels=2)
    gc.say("4-bit scores on rotated Q and K")
    gc.stage_and_chain(orc, q, k, v, do, cu, gc.full_window(T, Hq), hadamard=True, qk4=True)


def test_mx4_chunked_backward_identical():
    """Smallest workspace (several key-tile chunks) and the static scratch: bit-identical."""
    T, Hq, Hkv, d = 1536, 4, 2, 128
    cu = [0, 700, 705, 1300, 1301, 1536]
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=1620)
    a = gc.gpu_call(q, k, v, do, cu, qk4=True)
    b = gc.gpu_call(q, k, v, do, cu, qk4=True, store_budget=0)
    c = gc.gpu_call(q, k, v, do, cu, qk4=True, static_scratch=True)
    assert b["chunks"] > 1
    for nm in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[nm].view(np.uint8), b[nm].view(np.uint8)), nm
        assert np.array_equal(a[nm].view(np.uint8), c[nm].view(np.uint8)), nm
    gc.say("  4-bit scores: %d chunks and the static scratch bit-identical to one chunk" % b["chunks"])


@pytest.mark.parametrize("p", [96, 224])
def test_mx4_no_leakage(p):
    """Q, K, V perturbed (x16) from a block boundary p to the end of document 0, dO zero there,
    with the causal dQ prescale: every earlier row's O, dQ and every earlier key's dK, dV, and the
    other document, are bit-identical (the 4-bit copy is per token)."""
    T, Hq, Hkv, d = 520, 4, 2, 128
    cu = np.array([0, 300, T], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=1630)
    do = do.clone()
    do[p:300] = 0
    keep = np.ones(T, bool)
    keep[p:300] = False
    runs = []
    for scale in (1.0, 16.0):
        xs = []
        for x in (q, k, v):
            y = x.clone()
            y[p:300] = (y[p:300].to(torch.float32) * scale).to(torch.bfloat16)
            xs.append(y)
        runs.append(gc.gpu_call(*xs, do, cu, causal_dq=True, qk4=True))
    a, b = runs
    assert not np.array_equal(a["o"], b["o"])
    for nm in ("o", "dq", "dk", "dv"):
        assert np.array_equal(a[nm][keep], b[nm][keep]), nm
    gc.say("  4-bit scores, perturbation from offset %d: earlier rows bit-identical" % p)


def test_mx4_against_exact():
    """Accuracy of the 4-bit path on the 256-token workload against exact attention (reported;
    the pages give O cosine 0.9899 for their 4-bit scores on non-causal inputs)."""
    cu, shp, (q, k, v, do) = workloads.workload("single")
    g = gc.gpu_call(q, k, v, do, cu, qk4=True)
    f = lambda x: x.to(torch.float64).numpy()
    ref, dq, dk, dv, _ = exact_attention(f(q), f(k), f(v), cu, 1.0 / np.sqrt(shp.d), do=f(do))
    c = cosine(bits_to_f64(g["o"]), ref)
    cq, ck, cv = (cosine(bits_to_f64(g[n]), r) for n, r in (("dq", dq), ("dk", dk), ("dv", dv)))
    gc.say("  4-bit scores vs exact: O %.5f dQ %.5f dK %.5f dV %.5f" % (c, cq, ck, cv))
    assert c >= 0.98
