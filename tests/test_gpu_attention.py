"""GPU parity of the forward and backward against the oracle, through the C ABI.

Two levels, on the same seeded inputs:
  stage: the forward against the oracle's forward on the GPU's codes (bit-exact with the
         oracle's), and the backward against the oracle's backward on the same codes and the
         GPU's own LSE and D: cosine >= 0.9995 and, per element, max|diff| <= 2e-2 RMS plus
         the allowances derived from the arithmetic (one BF16 ulp, one E4M3 decision flip of a
         computed operand, the FP8 matrix instruction's accumulation bound); LSE within its
         bound; pi bit-exact;
  chain: the whole GPU call against the oracle's whole chain on the BF16 inputs: codes,
         scales, pi bit-exact; O, dQ, dK, dV cosine >= 0.9995 (spec bar)."""
import numpy as np
import pytest
import torch

from precision_causal_attention_token_amd import workloads
from tests.gpu_common import check_cosine, gpu_call, oracle_call, say, stage_check, token_mask
from tests.helpers import bits_to_f64, cosine, exact_attention

pytestmark = pytest.mark.gpu

# (name, T, Hq, Hkv, d, cu, tensor options)
SMALL = [
    ("single-256", 256, 2, 2, 64, [0, 256], {}),
    ("packed-d128-outliers", 1536, 4, 2, 128, [0, 700, 705, 1300, 1301, 1536], dict(outlier_channels=2)),
    ("offsets-gqa4-d64", 1200, 4, 1, 64, [9, 40, 41, 555, 1100], {}),
    ("ragged-d128-studentt", 1000, 2, 2, 128, [0, 129, 383, 385, 1000], dict(k_dist="student_t3")),
]


def _chain(orc, g, q, k, v, do, cu, causal_dq, docs=None, kv_heads=None, q_heads=None):
    r = oracle_call(orc, q, k, v, do, cu, causal_dq, docs=docs, kv_heads=kv_heads)
    for nm in ("q", "sq", "k", "sk", "v", "sv", "do", "sdo"):
        assert np.array_equal(g[nm], r[nm]), nm
    assert np.array_equal(g["pi"], r["pi"]), "pi"
    T = g["q"].shape[0]
    m = token_mask(cu, T, docs)
    qh = slice(None) if q_heads is None else q_heads
    kh = slice(None) if kv_heads is None else kv_heads
    check_cosine("O", g["o"][m][:, qh], r["o"][m][:, qh])
    check_cosine("dQ", g["dq"][m][:, qh], r["dq"][m][:, qh])
    check_cosine("dK", g["dk"][m][:, kh], r["dk"][m][:, kh])
    check_cosine("dV", g["dv"][m][:, kh], r["dv"][m][:, kh])


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("causal_dq", [False, True])
def test_small_parity(orc, case, causal_dq):
    name, T, Hq, Hkv, d, cu, opts = SMALL[case]
    say("parity %s causal_dq=%s" % (name, causal_dq))
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=500 + case, **opts)
    g = gpu_call(q, k, v, do, cu, causal_dq)
    stage_check(orc, g, cu, causal_dq)
    _chain(orc, g, q, k, v, do, cu, causal_dq)
    out = ~token_mask(cu, T)
    if out.any():
        assert not g["o"][out].any() and np.all(np.isinf(g["lse"][:, out]))
        assert not g["dq"][out].any() and not g["dk"][out].any() and not g["dv"][out].any()
        assert not g["D"][:, out].any()


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


@pytest.mark.parametrize("name", ["lognormal", "gqa", "long"])
def test_full_size_sampled_documents(orc, name):
    """Full-size workload on the GPU (the configuration the benchmark runs for `long`); the
    oracle recomputes a sample of documents (the three shortest and one of median length,
    each at most 4096 tokens) for two KV heads."""
    cu, shp, (q, k, v, do) = workloads.workload(name)
    say("full-size %s T=%d Hq=%d Hkv=%d d=%d docs=%d" % (name, shp.T, shp.Hq, shp.Hkv, shp.d, len(cu) - 1))
    g = gpu_call(q, k, v, do, cu, causal_dq=True)
    L = np.diff(cu)
    order = [i for i in np.argsort(L, kind="stable") if L[i] <= 4096]
    docs = sorted(set(order[:3] + [order[len(order) // 2]]))
    kv = [0, shp.Hkv - 1]
    grp = shp.Hq // shp.Hkv
    qh = [h for h in range(shp.Hq) if h // grp in kv]
    say("  sampled docs %s (lengths %s), kv heads %s" % (docs, L[docs].tolist(), kv))
    stage_check(orc, g, cu, True, docs=docs, kv_heads=kv, q_heads=qh)
    _chain(orc, g, q, k, v, do, cu, True, docs=docs, kv_heads=kv, q_heads=qh)
