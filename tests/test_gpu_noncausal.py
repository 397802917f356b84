"""GPU parity of the non-causal variant (every key of a row's document visible; batched
attention is the case of equal-length documents) against the oracle, through the C ABI: the
same stage and chain checks as the causal cases (tests/gpu_common.py) with the non-causal mask,
running maxima from the document's last key tile down, and every key tile's dQ partial in each
row's FP16 sum."""
import numpy as np
import pytest
import torch

import precision_causal_attention_token_amd as fl
from precision_causal_attention_token_amd import workloads
from tests.gpu_common import doc_window, full_window, gpu_call, say, stage_and_chain, token_mask
from tests.helpers import bits_to_f64, cosine, exact_attention

pytestmark = pytest.mark.gpu

# (name, T, Hq, Hkv, d, cu, tensor options)
NC_SMALL = [
    ("nc-single-256", 256, 2, 2, 64, [0, 256], {}),
    ("nc-batched-4x512-d128", 2048, 4, 4, 128, [0, 512, 1024, 1536, 2048], {}),
    ("nc-packed-d128-outliers", 1536, 4, 2, 128, [0, 700, 705, 1300, 1301, 1536], dict(outlier_channels=2)),
    ("nc-offsets-gqa4-d64-empty", 1200, 4, 1, 64, [9, 40, 41, 555, 555, 1100], {}),
    ("nc-ragged-d64-studentt", 1000, 2, 1, 64, [0, 129, 383, 385, 1000], dict(k_dist="student_t3")),
    ("nc-one-4096-d128-8wave", 4096, 2, 2, 128, [0, 4096], {}),
    # longest document >= 4x the average: the forward takes its units dynamically
    ("nc-skewed-dynamic-d128", 2560, 4, 2, 128, [0, 2048] + [2048 + 64 * i for i in range(1, 9)], {}),
]


@pytest.mark.parametrize("case", range(len(NC_SMALL)), ids=[c[0] for c in NC_SMALL])
def test_non_causal_parity(orc, case):
    name, T, Hq, Hkv, d, cu, opts = NC_SMALL[case]
    say("non-causal parity %s" % name)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=900 + case, **opts)
    release = gpu_call(q, k, v, do, cu, causal=False)
    stage_and_chain(orc, q, k, v, do, cu, full_window(T, Hq), release=release, causal=False)
    out = ~token_mask(cu, T)
    if out.any():
        g = release
        assert not g["o"][out].any() and np.all(np.isinf(g["lse"][:, out]))
        assert not g["dq"][out].any() and not g["dk"][out].any() and not g["dv"][out].any()


def test_non_causal_against_exact():
    """Batched non-causal attention (four 512-token sequences) against exact attention on the
    unquantised inputs: O cosine >= 0.998 (gradients reported)."""
    T, H, d = 2048, 4, 128
    cu = [0, 512, 1024, 1536, 2048]
    q, k, v, do = workloads.tensors(T, H, H, d, seed=950)
    g = gpu_call(q, k, v, do, cu, causal=False)
    f = lambda x: x.to(torch.float64).numpy()
    ref, dq, dk, dv, _ = exact_attention(f(q), f(k), f(v), cu, 1.0 / np.sqrt(d), do=f(do), causal=False)
    c = cosine(bits_to_f64(g["o"]), ref)
    cq, ck, cv = (cosine(bits_to_f64(g[n]), r) for n, r in (("dq", dq), ("dk", dk), ("dv", dv)))
    say("  non-causal vs exact: O %.5f dQ %.5f dK %.5f dV %.5f" % (c, cq, ck, cv))
    assert c >= 0.998


def test_non_causal_chunked_backward_bit_identical():
    """The non-causal backward with the smallest workspace (many key-tile chunks, FP16 dQ sums
    carried between them) gives the same bits as one chunk."""
    T, Hq, Hkv, d = 4096, 4, 2, 128
    cu = np.array([0, 1500, 1501, 1700, 3000, 4096], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=960)
    one = gpu_call(q, k, v, do, cu, store_budget=1 << 40, causal=False)
    many = gpu_call(q, k, v, do, cu, store_budget=0, causal=False)
    say("non-causal chunked backward: %d chunk(s) vs %d chunks" % (one["chunks"], many["chunks"]))
    assert one["chunks"] == 1 and many["chunks"] >= 4
    for nm in ("dq", "dk", "dv", "pi"):
        assert np.array_equal(one[nm], many[nm]), nm


def test_non_causal_long_document_tail(orc):
    """A 16384-token document (128 key tiles): the last 128 query rows of one head, all keys;
    every row's dQ sums all 128 key tiles' FP16 partials."""
    T, Hq, Hkv, d = 16384, 2, 1, 128
    cu = np.array([0, T], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=970)
    stage_and_chain(orc, q, k, v, do, cu, doc_window(cu, 0, (1, 2), tail_blocks=4), tail=True, causal=False)


def test_non_causal_dynamic_schedule_8wave(orc):
    """A 16384-token document and three empty ones (longest = 4x the average: a dynamic list, on
    the 8-wave forward): the last 128 rows of one head against the oracle; the forward run twice on
    the same list (its counters cleared by the first) gives the same bits and leaves them cleared."""
    T, Hq, Hkv, d = 16384, 2, 1, 128
    cu = np.array([0, T, T, T, T], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=975)
    stage_and_chain(orc, q, k, v, do, cu, doc_window(cu, 0, (1, 2), tail_blocks=4), tail=True, causal=False)
    dev = torch.device("cuda:0")
    cu_d = torch.as_tensor(cu).to(dev)
    lists = fl.Lists(cu_d, T, causal=False)
    assert int(lists.fwd[3].item()) != 0  # marked dynamic
    qz, kz, vz = fl.quantize([x.to(dev) for x in (q, k, v)], cu_d)
    runs = [fl.fwd(qz, kz, vz, cu_d, lists.fwd, causal=False) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    ctr = lists.fwd[(16 + 16 * ((T + 127) // 128 + len(cu) - 1)) // 4:][:16]
    assert not ctr.any()
    say("  dynamic forward: two runs on one list bit-identical, counters cleared")


def test_non_causal_with_hadamard_rotation(orc):
    """Both options together: rotated Q, K on non-causal attention, stage and chain checks."""
    T, Hq, Hkv, d = 1100, 4, 2, 128
    cu = [0, 200, 201, 700, 1100]
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=980, outlier_channels=2)
    stage_and_chain(orc, q, k, v, do, cu, full_window(T, Hq), causal=False, hadamard=True)


def test_non_causal_static_scratch_matches_workspace():
    """flamia_bwd_static on non-causal attention gives the bits of flamia_bwd."""
    T, Hq, Hkv, d = 3000, 4, 2, 64
    cu = np.array([0, 1000, 1001, 2500, 3000], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=990)
    a = gpu_call(q, k, v, do, cu, causal=False)
    b = gpu_call(q, k, v, do, cu, causal=False, static_scratch=True)
    for nm in ("dq", "dk", "dv", "pi"):
        assert np.array_equal(a[nm], b[nm]), nm
