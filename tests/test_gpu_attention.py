"""GPU parity of the forward and backward against the oracle, through the C ABI.

Every case runs the product library and the parity tests' debug variant (same kernels plus
per-pair dumps; outputs compared bit for bit), then, in a window of rows, keys and heads
(tests/gpu_common.py):
  stage: forward and backward scores bit-identical (masks included); scores and D - dP within
         the FP8 instruction's accumulation bound of the exact dot products; running maxima equal
         to the FP32 recomputation; every E4M3 decision (probability codes, Phat / dShat codes
         and block exponents) equal to the oracle's rounding of the value the method defines,
         or at a rounding boundary (counted); O, LSE, dQ, dK, dV against the oracle's replay on
         those decisions at max|diff| <= 2e-2 RMS + one BF16 ulp; pi bit-exact;
  chain: the whole GPU call against the oracle's own chain on the BF16 inputs: codes, scales,
         pi bit-exact, cosine >= 0.9995, every element beyond 2e-2 RMS + 1 ulp named with the
         part of its difference that the decisions account for."""
import numpy as np
import pytest
import torch

from precision_causal_attention_token_amd import workloads
from tests.gpu_common import (doc_window, full_window, gpu_call, say, stage_and_chain, token_mask)
from tests.helpers import bits_to_f64, cosine, exact_attention

pytestmark = pytest.mark.gpu

# (name, T, Hq, Hkv, d, cu, tensor options)
SMALL = [
    ("single-256", 256, 2, 2, 64, [0, 256], {}),
    ("packed-d128-outliers", 1536, 4, 2, 128, [0, 700, 705, 1300, 1301, 1536], dict(outlier_channels=2)),
    ("offsets-gqa4-d64-empty", 1200, 4, 1, 64, [9, 40, 41, 555, 555, 1100], {}),
    ("ragged-d128-studentt", 1000, 2, 2, 128, [0, 129, 383, 385, 1000], dict(k_dist="student_t3")),
    # one 4096-token document: documents average >= 4096 tokens, so the forward runs its 8-wave
    # shape (the one the 65536-token benchmark uses) over 32 key tiles
    ("one-4096-d128-8wave", 4096, 2, 2, 128, [0, 4096], {}),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("causal_dq", [False, True])
def test_small_parity(orc, case, causal_dq):
    name, T, Hq, Hkv, d, cu, opts = SMALL[case]
    if name.endswith("8wave") and causal_dq:
        pytest.skip("one prescale mode suffices for the forward-shape case")
    say("parity %s causal_dq=%s" % (name, causal_dq))
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=500 + case, **opts)
    release = gpu_call(q, k, v, do, cu, causal_dq)
    stage_and_chain(orc, q, k, v, do, cu, full_window(T, Hq), causal_dq, release=release)
    out = ~token_mask(cu, T)
    if out.any():
        g = release
        assert not g["o"][out].any() and np.all(np.isinf(g["lse"][:, out]))
        assert not g["dq"][out].any() and not g["dk"][out].any() and not g["dv"][out].any()
        assert not g["D"][:, out].any()


def test_forward_shapes_bit_identical():
    """The forward's two workgroup shapes (4 waves / 128-query units below 4096 tokens per
    document on average, else 8 waves / 256-query units) compute the same values: one 1000-token
    document alone (4-wave shape) and padded to T = 4096 with rows outside every document
    (8-wave shape) give bit-identical O, LSE and gradients on its rows."""
    T0, H, d = 1000, 2, 128
    q, k, v, do = workloads.tensors(4096, H, H, d, seed=530)
    small = gpu_call(q[:T0], k[:T0], v[:T0], do[:T0], [0, T0])
    padded = gpu_call(q, k, v, do, [0, T0])
    for nm in ("o", "dq", "dk", "dv"):
        assert np.array_equal(small[nm], padded[nm][:T0]), nm
    assert np.array_equal(small["lse"], padded["lse"][:, :T0])
    say("  forward shapes: 4-wave and 8-wave results bit-identical on 1000 rows")


def test_single_workload_against_exact():
    """North-star yardstick on the 256-token workload: O cosine >= 0.998 against exact
    attention on the unquantised inputs (gradients reported)."""
    cu, shp, (q, k, v, do) = workloads.workload("single")
    g = gpu_call(q, k, v, do, cu, False)
    f = lambda x: x.to(torch.float64).numpy()
    ref, dq, dk, dv, _ = exact_attention(f(q), f(k), f(v), cu, 1.0 / np.sqrt(shp.d), do=f(do))
    c = cosine(bits_to_f64(g["o"]), ref)
    cq, ck, cv = (cosine(bits_to_f64(g[n]), r) for n, r in (("dq", dq), ("dk", dk), ("dv", dv)))
    say("  vs exact: O %.5f dQ %.5f dK %.5f dV %.5f" % (c, cq, ck, cv))
    assert c >= 0.998


@pytest.mark.parametrize("name,causal_dq", [("lognormal", True), ("gqa", True), ("gqa", False), ("long", True)])
def test_full_size_sampled_documents(orc, name, causal_dq):
    """Full-size workload on the GPU; stage and chain checks on a sample of documents (the
    shortest, and one of median length, each at most 4096 tokens) for the query heads of one
    KV head.  The GQA workload runs with the causal dQ prescale off and on."""
    cu, shp, (q, k, v, do) = workloads.workload(name)
    say("full-size %s T=%d Hq=%d Hkv=%d d=%d docs=%d causal_dq=%s" % (name, shp.T, shp.Hq, shp.Hkv, shp.d,
                                                                   len(cu) - 1, causal_dq))
    release = gpu_call(q, k, v, do, cu, causal_dq=causal_dq)
    L = np.diff(cu)
    order = [i for i in np.argsort(L, kind="stable") if L[i] <= 4096]
    docs = sorted(set([order[0], order[len(order) // 2]]))
    grp = shp.Hq // shp.Hkv
    g_kv = shp.Hkv - 1
    for doc in docs:
        say(" document %d (%d tokens), query heads of KV head %d" % (doc, L[doc], g_kv))
        stage_and_chain(orc, q, k, v, do, cu, doc_window(cu, doc, (g_kv * grp, (g_kv + 1) * grp)), causal_dq,
                        release=release)


@pytest.mark.parametrize("which", ["longest", "shortest-long"])
def test_long_workload_bench_configuration(orc, which):
    """The 65536-token workload in the benchmark's configuration (default dQ prescale, 8-wave
    forward), on the tail of its longest document (29368 tokens, 230 key tiles) and of its
    shortest long one (16853 tokens): the last 128 query rows (4 blocks) of the last head, all
    keys of the document.  dQ of those rows sums every key tile's FP16 partial; dK, dV of those
    keys see every query after them."""
    cu, shp, (q, k, v, do) = workloads.workload("long")
    L = np.diff(np.asarray(cu, np.int64))
    if which == "longest":
        doc = int(np.argmax(L))
    else:
        doc = int(np.argmin(np.where(L > 4096, L, np.iinfo(np.int64).max)))
    h = shp.Hq - 1
    say("long workload: document %d (%d tokens), head %d, last 4 query blocks" % (doc, L[doc], h))
    stage_and_chain(orc, q, k, v, do, cu, doc_window(cu, doc, (h, h + 1), tail_blocks=4), False, tail=True)


def test_single_long_document_tail(orc):
    """Extreme packing, one 131072-token document (1024 key tiles), default dQ prescale: stage
    and chain checks on the last 128 rows of the last head (dQ an FP16 sum over 1024 key-tile
    partials)."""
    cu, shp, (q, k, v, do) = workloads.workload("onedoc")
    h = shp.Hq - 1
    say("single %d-token document, head %d, last 128 rows" % (shp.T, h))
    stage_and_chain(orc, q, k, v, do, cu, doc_window(cu, 0, (h, h + 1), tail_blocks=4), False, tail=True)
