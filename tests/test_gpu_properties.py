"""GPU properties that hold at any size: causal leakage exactly zero (jaehun.me review §4.5,
read per the design notes: perturbation from a 32-token block boundary on, dO zeroed there,
causal dQ scale), document isolation, run-to-run bit reproducibility, one-token documents
(O = BF16(0 + deq V) and dV = BF16(0 + deq dO) bit-exactly)."""
import numpy as np
import pytest
import torch

import precision_causal_attention_token_amd as fl
from precision_causal_attention_token_amd import workloads
from tests.gpu_common import full_window, gpu_call, say, stage_and_chain, token_mask
from tests.helpers import bf16_bits, bits_to_f64, dequant

pytestmark = pytest.mark.gpu


def _perturb(x, a, b, scale):
    y = x.clone()
    y[a:b] = (y[a:b].to(torch.float32) * scale).to(torch.bfloat16)
    return y


@pytest.mark.parametrize("d,b0", [(128, 160), (64, 32)])
def test_leakage_is_zero(d, b0):
    T, Hq, Hkv = 1200, 4, 2
    cu = np.array([0, 700, 1200], np.int32)
    a, b = 0, 700
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=700 + d)
    do = do.clone()
    do[a + b0:b] = 0
    say("leakage d=%d b0=%d" % (d, b0))
    base = gpu_call(q, k, v, do, cu, causal_dq=True)
    pert = gpu_call(*(_perturb(x, a + b0, b, 1024.0) for x in (q, k, v)), do, cu, causal_dq=True)
    keep = np.ones(T, bool)
    keep[a + b0:b] = False
    assert not np.array_equal(base["o"], pert["o"])
    for nm in ("o", "dq", "dk", "dv"):
        same = np.array_equal(base[nm][keep], pert[nm][keep])
        say("  %s earlier rows bit-identical: %s" % (nm, same))
        assert same, nm
    assert np.array_equal(base["lse"][:, keep], pert["lse"][:, keep])
    # the sequence-wide default prescale does depend on the perturbed tokens
    base_d = gpu_call(q, k, v, do, cu, causal_dq=False)
    pert_d = gpu_call(*(_perturb(x, a + b0, b, 1024.0) for x in (q, k, v)), do, cu, causal_dq=False)
    moved = not np.array_equal(base_d["pi"][:, keep], pert_d["pi"][:, keep])
    say("  default prescale moved: %s; dQ of earlier rows changed: %s"
        % (moved, not np.array_equal(base_d["dq"][keep], pert_d["dq"][keep])))
    assert moved


def test_document_isolation():
    """Scaling one document x1e4 (jaehun.me review §4.7) leaves every output of the other
    documents bit-identical (causal dQ scale)."""
    T, H, d = 1500, 2, 128
    cu = np.array([0, 400, 1000, 1500], np.int32)
    q, k, v, do = workloads.tensors(T, H, H, d, seed=710)
    base = gpu_call(q, k, v, do, cu, causal_dq=True)
    pert = gpu_call(*(_perturb(x, 400, 1000, 1e4) for x in (q, k, v, do)), cu, causal_dq=True)
    keep = np.ones(T, bool)
    keep[400:1000] = False
    for nm in ("o", "dq", "dk", "dv"):
        assert np.array_equal(base[nm][keep], pert[nm][keep]), nm


def test_bitwise_reproducible():
    cu, shp, (q, k, v, do) = workloads.workload("lognormal")
    say("determinism on lognormal workload")
    r1 = gpu_call(q, k, v, do, cu, causal_dq=False)
    r2 = gpu_call(q, k, v, do, cu, causal_dq=False)
    for nm in r1:
        assert np.array_equal(r1[nm], r2[nm]), nm


def _check_one_token_closed_form(g):
    """O = BF16(0 + deq V) and dV = BF16(0 + deq dO), bit for bit.  The sums start from +0, so
    an E4M3 negative zero (code 0x80) contributes -0 and leaves +0 (IEEE addition), as in the
    oracle."""
    vd = dequant(g["v"], g["sv"]) + 0.0
    assert np.array_equal(g["o"], bf16_bits(torch.from_numpy(vd).to(torch.bfloat16)))
    dod = dequant(g["do"], g["sdo"]) + 0.0
    assert np.array_equal(g["dv"], bf16_bits(torch.from_numpy(dod).to(torch.bfloat16)))


def test_one_token_documents(orc):
    """O = BF16(0 + deq V) and dV = BF16(0 + deq dO) bit-exactly; dQ and dK are zero in exact
    arithmetic (D = dP) and stay within the stage bar (accumulation-level values)."""
    T, H, d = 512, 2, 128
    cu = workloads.cu_seqlens([1] * T)
    q, k, v, do = workloads.tensors(T, H, H, d, seed=720)
    g = gpu_call(q, k, v, do, cu)
    _check_one_token_closed_form(g)
    stage_and_chain(orc, q, k, v, do, cu, full_window(T, H), release=g, zero_in_exact=("dQ", "dK"))


def test_one_token_documents_full_size(orc):
    """Extreme packing at full size, 131072 one-token documents x 8 heads: O = BF16(0 + deq V)
    and dV = BF16(0 + deq dO) bit-exactly for every token; stage and chain checks (dQ, dK zero in
    exact arithmetic) on 1024 consecutive documents in the middle of the call, all heads."""
    cu, shp, (q, k, v, do) = workloads.workload("tokens")
    say("one-token documents: T=%d H=%d d=%d" % (shp.T, shp.Hq, shp.d))
    g = gpu_call(q, k, v, do, cu)
    _check_one_token_closed_form(g)
    a = shp.T // 2
    win = dict(row_lo=a, row_hi=a + 1024, key_lo=a, key_hi=a + 1024, head_lo=0, head_hi=shp.Hq)
    stage_and_chain(orc, q, k, v, do, cu, win, release=g, zero_in_exact=("dQ", "dK"))


@pytest.mark.parametrize("causal_dq", [False, True])
def test_chunked_backward_bit_identical(causal_dq):
    """A backward whose dShat store holds only two of the largest key tiles (the smallest
    workspace: many chunks, FP16 dQ sums carried between them in the dQ rows) gives the same
    bits as one chunk: the backward list keeps each document's key tiles in ascending order
    across chunks, so every FP16 sum adds the same partials in the same order."""
    T, Hq, Hkv, d = 4096, 4, 2, 128
    cu = np.array([0, 1500, 1501, 1700, 3000, 4096], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=730)
    one = gpu_call(q, k, v, do, cu, causal_dq, store_budget=1 << 40)
    many = gpu_call(q, k, v, do, cu, causal_dq, store_budget=0)
    say("chunked backward: %d chunk(s) vs %d chunks" % (one["chunks"], many["chunks"]))
    assert one["chunks"] == 1 and many["chunks"] >= 4
    for nm in ("dq", "dk", "dv", "pi"):
        assert np.array_equal(one[nm], many[nm]), nm


def test_max_doc_len_bound():
    """The backward's bound of the longest document (fewer chunk launches): with the true longest
    length the outputs and the chunk count are those of the unbounded call, in the smallest
    workspace (several chunks) and in a one-chunk store; a bound so low that the launched chunks
    cannot hold the documents makes the call report status 3 (the gradient passes do not run)."""
    T, Hq, Hkv, d = 4096, 4, 2, 128
    cu = np.array([0, 1500, 1501, 1700, 3000, 4096], np.int32)
    q, k, v, do = workloads.tensors(T, Hq, Hkv, d, seed=731)
    for budget in (0, 1 << 40):
        free = gpu_call(q, k, v, do, cu, True, store_budget=budget)
        bound = gpu_call(q, k, v, do, cu, True, store_budget=budget, max_doc_len=1500)
        assert free["chunks"] == bound["chunks"]
        for nm in ("dq", "dk", "dv", "pi"):
            assert np.array_equal(free[nm], bound[nm]), nm
        say("max_doc_len = 1500, store budget %d: %d chunk(s), bit-identical" % (budget, free["chunks"]))
    # too low: launches for documents of at most 200 tokens, the smallest store
    dev = torch.device("cuda:0")
    cu_d = torch.as_tensor(cu).to(dev)
    lists = fl.Lists(cu_d, T, True)
    qz, kz, vz = fl.quantize([x.to(dev) for x in (q, k, v)], cu_d)
    o, lse = fl.fwd(qz, kz, vz, cu_d, lists.fwd)
    dc, dsc, D = fl.quantize_do(do.to(dev), o, cu_d)
    ws = torch.empty(fl.bwd_workspace_bytes(len(cu) - 1, T, Hq, d, 0), dtype=torch.uint8, device=dev)
    dq, dk, dv = fl.bwd(qz, kz, vz, (dc, dsc), lse, D, cu_d, lists, workspace=ws, max_doc_len=200)
    torch.cuda.synchronize()
    status, _ = fl.bwd_status(ws)
    assert status == 3
    say("max_doc_len = 200 below the 1500-token document: status %d" % status)


def test_chunked_backward_long_document():
    """The 65536-token workload's documents with a 1 GiB store (several chunks, one 29368-token
    document spread over them) against one chunk: dQ, dK, dV bit-identical."""
    cu, shp, (q, k, v, do) = workloads.workload("long")
    one = gpu_call(q, k, v, do, cu, False, store_budget=1 << 40)
    many = gpu_call(q, k, v, do, cu, False, store_budget=1 << 30)
    say("long workload: %d chunk(s) vs %d chunks" % (one["chunks"], many["chunks"]))
    assert one["chunks"] == 1 and many["chunks"] >= 8
    for nm in ("dq", "dk", "dv"):
        assert np.array_equal(one[nm], many[nm]), nm
