"""GPU parity of the fused reorder + block pooling (+ INT8) pass, the mask
build from pooled sums, and the online axis-order choice (SICS), through the
C ABI against the CPU oracle on the same seeded inputs.

Everything here is bit-exact: reordered rows, fp32 block sums (a fixed
sequential order), INT8 codes and scales, CSR, the fp32 SICS scores (a fixed
operation sequence) and the chosen order codes.
"""
import numpy as np
import pytest
import torch

from test_gpu_parity import (MASK_CASES, _bits, _np, _say, case, mask_params,
                             oracle_reorder)

pytestmark = pytest.mark.gpu


def _natural_host(c, name):
    return c["host"][name]


# ----------------------------------------------- fused reorder + pool + int8
@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_permute_pool_bit_exact(bsa_gpu, orc, cid):
    c = case(cid)
    cfg = c["cfg"]
    F, H, W = cfg["F"], cfg["H"], cfg["W"]
    for name, B in (("Q", cfg["Bq"]), ("K", cfg["Bk"])):
        _say(f"[permute_pool cfg {cid} {name} B={B}]")
        xp, sums, (xq, sc) = bsa_gpu.permute_pool(c[name], c["orders_dev"], F, H, W, B, sums=True,
                                                  int8=True)
        # the same pass without the bf16 copy
        _, sums2, (xq2, sc2) = bsa_gpu.permute_pool(c[name], c["orders_dev"], F, H, W, B,
                                                    sums=True, int8=True, reordered=False)
        torch.cuda.synchronize()
        want = oracle_reorder(orc, c, name)
        assert np.array_equal(_bits(xp), want)
        ws = orc.block_sums(want, B)
        assert np.array_equal(_np(sums), ws)
        wq, wsc = orc.quantize_int8(want, B)
        assert np.array_equal(_np(sc), wsc)
        assert np.array_equal(_np(xq), wq)
        assert torch.equal(sums2, sums) and torch.equal(xq2, xq) and torch.equal(sc2, sc)


def test_permute_pool_matches_unfused_calls(bsa_gpu):
    """Fused outputs equal bsa_permute + bsa_quantize_int8 on the GPU, for
    the [G][N][d] natural layout (a strided view) and the sums alone."""
    c = case(2)
    cfg = c["cfg"]
    F, H, W, B = cfg["F"], cfg["H"], cfg["W"], cfg["Bq"]
    view = c["V"].transpose(0, 1).contiguous().transpose(0, 1)
    xp, sums, (xq, sc) = bsa_gpu.permute_pool(view, c["orders_dev"], F, H, W, B, sums=True,
                                              int8=True)
    xp_ref = bsa_gpu.permute(view, c["orders_dev"], F, H, W, 0)
    xq_ref, sc_ref = bsa_gpu.quantize_int8(xp_ref, B)
    _, sums_only, none8 = bsa_gpu.permute_pool(view, c["orders_dev"], F, H, W, B, sums=True)
    torch.cuda.synchronize()
    assert none8 is None
    assert torch.equal(xp, xp_ref) and torch.equal(xq, xq_ref) and torch.equal(sc, sc_ref)
    assert torch.equal(sums_only, sums)


@pytest.mark.parametrize("cid,over,rho", MASK_CASES)
def test_build_mask_pooled_bit_exact(bsa_gpu, orc, cid, over, rho):
    c = case(cid)
    cfg = dict(c["cfg"], **over)
    F, H, W = cfg["F"], cfg["H"], cfg["W"]
    p = mask_params(bsa_gpu, cfg, rho)
    _say(f"[mask_pooled cfg {cid} {over} rho={rho}] Bq={p.Bq} Bk={p.Bk} score={p.score}")
    _, sq, _ = bsa_gpu.permute_pool(c["Q"], c["orders_dev"], F, H, W, p.Bq, sums=True,
                                    reordered=False)
    _, sk, _ = bsa_gpu.permute_pool(c["K"], c["orders_dev"], F, H, W, p.Bk, sums=True,
                                    reordered=False)
    rp, ci, nnz = bsa_gpu.build_mask_pooled(sq, sk, c["orders_dev"], F, H, W, p)
    torch.cuda.synchronize()
    oq, ok_ = oracle_reorder(orc, c, "Q"), oracle_reorder(orc, c, "K")
    wrp, wci = orc.build_mask(oq, ok_, F, H, W, c["orders"], p.Bq, p.Bk, p.score, p.rho_num,
                              p.rho_den, p.force_diag, p.win_T, p.win_r0)
    n = int(_np(nnz)[0])
    _say(f"  nnz={n}")
    assert n == int(wrp[-1])
    assert np.array_equal(_np(rp), wrp)
    assert np.array_equal(_np(ci)[:n], wci)


@pytest.mark.parametrize("int8", [False, True])
def test_layer_forward_fused_equals_unfused(bsa_gpu, int8):
    """The fused chain feeds the attention the same bytes as the unfused one,
    so the layer outputs are identical."""
    c = case(3)
    cfg = c["cfg"]
    G, F, H, W, d = cfg["G"], cfg["F"], cfg["H"], cfg["W"], cfg["d"]
    p = mask_params(bsa_gpu, cfg)
    _say(f"[layer fused vs unfused cfg 3 int8={int8}]")
    outs = []
    for fused in (False, True):
        plan = bsa_gpu.LayerPlan(G, F, H, W, d, "cuda", p, int8=int8, fused=fused)
        O = bsa_gpu.layer_forward(plan, c["Q"], c["K"], c["V"], c["orders_dev"])
        torch.cuda.synchronize()
        outs.append((O.clone(), plan.row_ptr.clone(), plan.col_idx[: int(plan.nnz.item())].clone()))
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][2], outs[1][2])
    assert torch.equal(outs[0][0], outs[1][0])


# ----------------------------------------------------------- SICS orders
@pytest.mark.parametrize("cid,B", [(1, 64), (2, 64), (3, 128), (4, 128), (4, 64)])
def test_order_scores_bit_exact(bsa_gpu, orc, cid, B):
    c = case(cid)
    cfg = c["cfg"]
    G, F, H, W, d = cfg["G"], cfg["F"], cfg["H"], cfg["W"], cfg["d"]
    _say(f"[order_scores cfg {cid} B={B}]")
    sq = bsa_gpu.order_scores(c["Q"], F, H, W, B)
    sk = bsa_gpu.order_scores(c["K"], F, H, W, B)
    chosen = bsa_gpu.select_orders(sq, sk)
    chosen_q = bsa_gpu.select_orders(sq)
    torch.cuda.synchronize()
    wq = orc.sics_scores(_natural_host(c, "Q"), G, F, H, W, d, B)
    wk = orc.sics_scores(_natural_host(c, "K"), G, F, H, W, d, B)
    assert np.array_equal(_np(sq).view(np.uint32), wq.view(np.uint32))
    assert np.array_equal(_np(sk).view(np.uint32), wk.view(np.uint32))
    want = orc.select_orders(wq, wk)
    assert np.array_equal(_np(chosen), want)
    assert np.array_equal(_np(chosen_q), orc.select_orders(wq))
    agree = float(np.mean(want == c["orders"]))
    _say(f"  chosen {want.tolist()[:12]} planted {c['orders'].tolist()[:12]} agree={agree:.2f}")


@pytest.mark.parametrize("axis", ["F", "H", "W"])
def test_order_scores_planted_axis(bsa_gpu, orc, axis):
    """Tokens constant along one axis of extent B: the orders with that axis
    innermost score nb*B^2 and one of them is chosen; GPU == oracle."""
    B, d, G = 64, 128, 3
    dims = {"F": 3, "H": 5, "W": 7}
    dims[axis] = B
    F, H, W = dims["F"], dims["H"], dims["W"]
    N = F * H * W
    r = np.random.Generator(np.random.PCG64(77))
    base = r.standard_normal((F, H, W, G, d)).astype(np.float32)
    ax = "FHW".index(axis)
    X = np.repeat(np.take(base, [0], axis=ax), B, axis=ax).reshape(N, G, d)
    x = torch.from_numpy(X).cuda().to(torch.bfloat16)
    s = bsa_gpu.order_scores(x, F, H, W, B)
    o = bsa_gpu.select_orders(s)
    torch.cuda.synchronize()
    host = orc.f32_to_bf16(X)
    want = orc.sics_scores(host, G, F, H, W, d, B)
    assert np.array_equal(_np(s).view(np.uint32), want.view(np.uint32))
    winners = [i for i, nm in enumerate(["FHW", "FWH", "HFW", "HWF", "WFH", "WHF"])
               if nm[2] == axis]
    assert all(int(v) in winners for v in _np(o))
    nb = N // B
    assert np.all(np.abs(_np(s)[:, winners] - nb * B * B) <= 1e-4 * nb * B * B)


@pytest.mark.parametrize("d,B,N3", [(64, 128, (1, 3, 7)), (128, 64, (2, 3, 5)), (64, 64, (3, 5, 9))])
def test_order_scores_small_and_ragged(bsa_gpu, orc, d, B, N3):
    """N below one block, and ragged tails, both dtypes."""
    F, H, W = N3
    N, G = F * H * W, 2
    r = np.random.Generator(np.random.PCG64(78))
    X = r.standard_normal((N, G, d)).astype(np.float32)
    X[N // 2] = 0.0  # an all-zero token counts as the zero vector
    for dt in (torch.float32, torch.bfloat16):
        x = torch.from_numpy(X).cuda().to(dt)
        s = bsa_gpu.order_scores(x, F, H, W, B)
        torch.cuda.synchronize()
        host = orc.f32_to_bf16(X) if dt == torch.bfloat16 else X
        want = orc.sics_scores(host, G, F, H, W, d, B)
        assert np.array_equal(_np(s).view(np.uint32), want.view(np.uint32)), (dt, N3)


# ------------------------------------------- inverse reorder in the epilogue
@pytest.mark.parametrize("cid,int8,layout", [(2, False, "NGd"), (2, True, "NGd"), (3, False, "GNd"),
                                             (3, True, "NGd"), (5, False, "NGd")])
def test_forward_natural_equals_forward_then_scatter(bsa_gpu, orc, cid, int8, layout):
    """The forward with the inverse reorder fused into its epilogue gives,
    bit for bit, the reordered forward followed by bsa_permute(direction 1),
    for natural [N][G][d] and strided [G][N][d] outputs; lse lands at the
    natural token index."""
    c = case(cid)
    cfg = c["cfg"]
    G, F, H, W, d = cfg["G"], cfg["F"], cfg["H"], cfg["W"], cfg["d"]
    N = F * H * W
    p = mask_params(bsa_gpu, cfg) if cfg["mask"] != "static" else bsa_gpu.mask_params(
        cfg["Bq"], cfg["Bk"], 0, (30, 100), True)
    _say(f"[forward natural cfg {cid} int8={int8} {layout}]")
    plan = bsa_gpu.LayerPlan(G, F, H, W, d, "cuda", p, int8=int8, fused=True)
    plan.reorder_fused(c["Q"], c["K"], c["V"], c["orders_dev"])
    plan.build_mask_from_sums(c["orders_dev"])
    if layout == "NGd":
        out_nat = torch.empty((N, G, d), dtype=torch.bfloat16, device="cuda")
    else:
        out_nat = torch.empty((G, N, d), dtype=torch.bfloat16, device="cuda").transpose(0, 1)
    if int8:
        o_r, l_r = bsa_gpu.forward_int8(plan.Qq, plan.sQ, plan.Kq, plan.sK, plan.Vq, plan.sV,
                                        plan.row_ptr, plan.col_idx, p.Bq, p.Bk)
        o_n, l_n = bsa_gpu.forward_int8_natural(plan.Qq, plan.sQ, plan.Kq, plan.sK, plan.Vq,
                                                plan.sV, plan.row_ptr, plan.col_idx, p.Bq, p.Bk,
                                                c["orders_dev"], F, H, W, out=out_nat)
    else:
        o_r, l_r = bsa_gpu.forward(plan.Qp, plan.Kp, plan.Vp, plan.row_ptr, plan.col_idx, p.Bq, p.Bk)
        o_n, l_n = bsa_gpu.forward_natural(plan.Qp, plan.Kp, plan.Vp, plan.row_ptr, plan.col_idx,
                                           p.Bq, p.Bk, c["orders_dev"], F, H, W, out=out_nat)
    want = bsa_gpu.permute(o_r, c["orders_dev"], F, H, W, 1)
    torch.cuda.synchronize()
    assert torch.equal(o_n.view(torch.int16), want.view(torch.int16))
    # lse: reordered position r of head g -> natural token perm_g(r)
    lr, ln = _np(l_r), _np(l_n)
    for g in range(G):
        pm = orc.perm(int(c["orders"][g]), F, H, W)
        assert np.array_equal(ln[g, pm], lr[g])
