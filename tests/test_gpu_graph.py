"""The planned layer step under HIP graph capture.

layer_forward on a LayerPlan launches only library kernels on the current
stream into preallocated buffers (the library issues no memset, copy or
allocation of its own), so the whole step - reorder with block sums (and
INT8 codes), mask build, attention writing natural order, optionally the
first-order compensation - can be captured once and replayed.  Each test
captures the step, then replays it three times with new inputs written
eagerly between the replays, and checks every replay bit for bit against
the same step run eagerly on a second plan.
"""
import pytest
import torch

from test_gpu_parity import _say, case, mask_params

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("int8,compensate", [(False, False), (True, False), (False, True)])
def test_layer_forward_graph_replays(bsa_gpu, int8, compensate):
    c = case(3)
    cfg = c["cfg"]
    G, F, H, W, d = cfg["G"], cfg["F"], cfg["H"], cfg["W"], cfg["d"]
    p = mask_params(bsa_gpu, cfg)
    od = c["orders_dev"]
    _say(f"[graph replay int8={int8} compensate={compensate}]")
    Q0, K0, V0 = (c[x].cuda() for x in ("Q", "K", "V"))
    Qs, Ks, Vs = Q0.clone(), K0.clone(), V0.clone()
    plan = bsa_gpu.LayerPlan(G, F, H, W, d, "cuda", p, int8=int8, fused=True, compensate=compensate)
    ref = bsa_gpu.LayerPlan(G, F, H, W, d, "cuda", p, int8=int8, fused=True, compensate=compensate)
    # one eager pass on a side stream before capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bsa_gpu.layer_forward(plan, Qs, Ks, Vs, od)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = bsa_gpu.layer_forward(plan, Qs, Ks, Vs, od)
    torch.cuda.synchronize()
    for rep in range(3):
        # new inputs, written eagerly between the replays
        s = 1.0 + 0.25 * rep
        Qs.copy_(Q0 * s)
        Ks.copy_(K0 * (2.0 - 0.25 * rep))
        Vs.copy_(V0 * s)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got, got_lse = out.clone(), plan.lse.clone()
        want = bsa_gpu.layer_forward(ref, Qs, Ks, Vs, od)
        torch.cuda.synchronize()
        _say(f"  replay {rep}: equal={torch.equal(got.view(torch.int16), want.view(torch.int16))}")
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        assert torch.equal(got_lse, ref.lse)
        assert torch.equal(plan.col_idx, ref.col_idx) and torch.equal(plan.row_ptr, ref.row_ptr)
