"""bsa_build_mask_pooled_noalloc (the mask build with the library's fixed
device scratch instead of a caller workspace) against bsa_build_mask_pooled
(caller workspace), through the C ABI: two calls in a row on one stream, the
720p layer and then a smaller 2k-shaped one, each CSR bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _case(bsa, cid):
    from block_sparse_attention_inverse_amd import synth

    cfg = synth.config(cid)
    seed = synth.seed_of(cid)
    F, H, W, G, d = cfg["F"], cfg["H"], cfg["W"], cfg["G"], cfg["d"]
    orders = synth.make_orders(cfg, seed)
    od = torch.from_numpy(orders).cuda()
    Q, K, _ = synth.cast_inputs(cfg, *synth.make_qkv(cfg, orders, seed, device="cuda"))
    p = bsa.mask_params(cfg["Bq"], cfg["Bk"], 0, cfg.get("rho", (30, 100)), True)
    _, sq, _ = bsa.permute_pool(Q, od, F, H, W, p.Bq, sums=True, reordered=False)
    _, sk, _ = bsa.permute_pool(K, od, F, H, W, p.Bk, sums=True, reordered=False)
    return dict(F=F, H=H, W=W, G=G, d=d, od=od, p=p, sq=sq, sk=sk)


def test_noalloc_mask_matches_workspace_mask(bsa_gpu):
    from block_sparse_attention_inverse_amd import _lib

    lib = _lib.load()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for cid in (4, 2):  # the second call is smaller than the first
        c = _case(bsa_gpu, cid)
        F, H, W, G, d, p = c["F"], c["H"], c["W"], c["G"], c["d"], c["p"]
        print(f"[noalloc cfg {cid}] G={G} N={F * H * W}", flush=True)
        nq = -(-F * H * W // p.Bq)
        cap = bsa_gpu.mask_capacity(G, F, H, W, p)
        ws = torch.empty(bsa_gpu.mask_workspace(G, F, H, W, d, p), dtype=torch.uint8, device="cuda")
        outs = []
        for noalloc in (False, True):
            rp = torch.full((G * nq + 1,), -7, dtype=torch.int32, device="cuda")
            ci = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
            nnz = torch.full((1,), -7, dtype=torch.int32, device="cuda")
            if noalloc:
                rc = lib.bsa_build_mask_pooled_noalloc(_p(c["sq"]), _p(c["sk"]), G, F, H, W, d,
                                                       _p(c["od"]), ctypes.byref(p), _p(rp), _p(ci),
                                                       cap, _p(nnz), st)
            else:
                rc = lib.bsa_build_mask_pooled(_p(c["sq"]), _p(c["sk"]), G, F, H, W, d, _p(c["od"]),
                                               ctypes.byref(p), _p(rp), _p(ci), cap, _p(nnz), _p(ws),
                                               ws.numel(), st)
            _lib.check(rc)
            outs.append((rp, ci, nnz))
        torch.cuda.synchronize()
        (rp0, ci0, n0), (rp1, ci1, n1) = outs
        n = int(n0.item())
        assert n == int(n1.item()) and n > 0
        assert torch.equal(rp0, rp1)
        assert torch.equal(ci0[:n], ci1[:n])
        # the Python binding, into the same kind of caller buffers
        rp2, ci2, n2 = bsa_gpu.build_mask_pooled_noalloc(
            c["sq"], c["sk"], c["od"], F, H, W, p, torch.empty_like(rp0), torch.empty_like(ci0),
            torch.empty_like(n0))
        torch.cuda.synchronize()
        assert int(n2.item()) == n and torch.equal(rp2, rp0) and torch.equal(ci2[:n], ci0[:n])
        print(f"  nnz={n} equal", flush=True)
