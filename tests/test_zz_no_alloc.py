"""flamia_bwd_static (the backward that allocates nothing, on the library's static device
scratch) against flamia_bwd (caller workspace) through the C ABI: bit-identical dQ, dK, dV and
pi on two calls in a row, the second smaller than the first (the scratch keeps the first call's
contents), and a call too large for the scratch rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import precision_causal_attention_token_amd as fl
from precision_causal_attention_token_amd import workloads
from tests.gpu_common import say

pytestmark = pytest.mark.gpu


def _forward_state(T, Hq, Hkv, d, cu, seed):
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in workloads.tensors(T, Hq, Hkv, d, seed=seed))
    cu_d = torch.as_tensor(np.asarray(cu, np.int32)).to(dev)
    lists = fl.Lists(cu_d, T)
    qz, kz, vz = fl.quantize([q, k, v], cu_d)
    o, lse = fl.fwd(qz, kz, vz, cu_d, lists.fwd)
    dc, dsc, D = fl.quantize_do(do, o, cu_d)
    return (qz, kz, vz, (dc, dsc), lse, D, cu_d, lists)


@pytest.mark.parametrize("causal_dq", [False, True])
def test_static_scratch_backward_matches(causal_dq):
    cases = [
        ("8192 tokens, lognormal lengths, 8 heads, d=128", 8192, 8, 8, 128,
         workloads.cu_seqlens(workloads.doc_lengths("lognormal"))),
        ("1000 tokens, ragged with offsets, GQA 4:1, d=64", 1000, 4, 1, 64, [9, 40, 41, 555, 555, 1000]),
    ]
    for i, (name, T, Hq, Hkv, d, cu) in enumerate(cases):
        say("static-scratch backward, call %d: %s, causal_dq=%s" % (i + 1, name, causal_dq))
        st = _forward_state(T, Hq, Hkv, d, cu, seed=740 + i)
        need = fl.bwd_workspace_bytes(len(cu) - 1, T, Hq, d, 0)
        assert need <= (64 << 20)
        ws = torch.empty(fl.bwd_workspace_bytes(len(cu) - 1, T, Hq, d), dtype=torch.uint8, device="cuda:0")
        ref = fl.bwd(*st, None, causal_dq, want_pi=True, workspace=ws)
        got = fl.bwd(*st, None, causal_dq, want_pi=True, static_scratch=True)
        torch.cuda.synchronize()
        for nm, a, b in zip(("dq", "dk", "dv", "pi"), got, ref):
            assert torch.equal(a, b), (name, nm)
        say("  dQ, dK, dV, pi bit-identical to flamia_bwd")


def test_static_scratch_rejects_large_calls():
    lib = fl.load_library()
    a = fl._BwdArgs()
    a.T, a.Hq, a.Hkv, a.d, a.n_docs = 65536, 16, 16, 128, 5
    assert fl.bwd_workspace_bytes(5, 65536, 16, 128, 0) > (64 << 20)
    assert lib.flamia_bwd_static(ctypes.byref(a), None) == 6       # FLAMIA_ERR_SCRATCH, nothing launched
    assert lib.flamia_status_str(6) == b"call too large for the static scratch"
