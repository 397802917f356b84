"""The training call captured in a HIP graph (torch.cuda.CUDAGraph over the library's calls on the
current stream): every replay gives the eager call's outputs bit for bit, with eager calls and
synchronisations between the replays.  Nothing in the call records a memset (the backward's
prologue clears its own counters), so replays after the first start from the same state."""
import numpy as np
import pytest
import torch

import precision_causal_attention_token_amd as fl
from precision_causal_attention_token_amd import workloads
from tests.gpu_common import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant", ["default", "causal_dq_chunked", "noncausal_dynamic"])
def test_graph_replays_match_eager(variant):
    """noncausal_dynamic: a skewed non-causal call, whose forward takes its units from the list's
    counters (cleared by each run for the next)."""
    T, Hq, Hkv, d = 1536, 4, 2, 128
    causal = variant != "noncausal_dynamic"
    cu = np.array([0, 700, 705, 1300, 1301, 1536] if causal else [0, 1280] + [1280 + 32 * i for i in range(1, 9)],
                  np.int32)
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in workloads.tensors(T, Hq, Hkv, d, seed=1700))
    cu_d = torch.as_tensor(cu).to(dev)
    lists = fl.Lists(cu_d, T, causal)  # built once per micro-batch, outside the graph
    if not causal:
        assert int(lists.fwd[3].item()) != 0  # marked dynamic
    causal_dq = variant == "causal_dq_chunked"
    budget = 0 if variant == "causal_dq_chunked" else fl.DEFAULT_STORE_BYTES
    ws = torch.empty(fl.bwd_workspace_bytes(len(cu) - 1, T, Hq, d, budget), dtype=torch.uint8, device=dev)
    names = ("o", "lse", "dq", "dk", "dv")

    def call():
        qz, kz, vz = fl.quantize([q, k, v], cu_d)
        o, lse = fl.fwd(qz, kz, vz, cu_d, lists.fwd, causal=causal)
        dc, dsc, D = fl.quantize_do(do, o, cu_d)
        dq, dk, dv = fl.bwd(qz, kz, vz, (dc, dsc), lse, D, cu_d, lists, None, causal_dq, workspace=ws, causal=causal)
        return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)

    eager = {n: x.clone() for n, x in call().items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one call on the capture stream before capturing
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = call()
    torch.cuda.synchronize()
    for i in range(3):
        again = call()  # eager work between the replays
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(again[n], eager[n]), ("eager", i, n)
        graph.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(out[n], eager[n]), ("replay", i, n)
    status, chunks = fl.bwd_status(ws)
    assert status == 0
    say("graph (%s): 3 replays bit-identical to the eager call (%d key-tile chunk(s))" % (variant, chunks))
