"""GPU parity on seeded random shapes.

Each case draws a small F x H x W grid (down to a few tokens, so blocks are
ragged and sequences can be shorter than one block), a head count, a head
dimension, a block shape, per-head axis orders and mask parameters (DOT or
COSINE scores, the Top-K share, the diagonal, a temporal window), then checks
on the same seeded inputs:

* the mask build against the oracle's, bit for bit (row_ptr, col_idx, nnz);
* the bf16 forward with natural-order output, every row, against the oracle's
  fp64 masked attention (rel-L2 <= 1e-2, max |diff| <= 2e-2, LSE within 1e-3);
* the first-order compensation applied to that output, against the oracle's
  compensated attention on every second row;
* the INT8 forward on the same mask, every q-block, against the oracle's INT8
  emulation on its own quantisation of the same bf16 values;
* the order choice (SICS scores, bit for bit) and the calibration's block
  statistics of the dense map.
"""
import numpy as np
import pytest
import torch

from test_gpu_coverage import _bf16, _compare, _int8_all_blocks, _np, _say

pytestmark = pytest.mark.gpu

LSE_ABS = 1e-3
NCASES = 10


def _draw(k):
    r = np.random.Generator(np.random.PCG64(5100 + k))
    F, H, W = int(r.integers(1, 7)), int(r.integers(2, 17)), int(r.integers(3, 61))
    return dict(
        F=F, H=H, W=W, N=F * H * W, G=int(r.integers(1, 4)), d=int(r.choice([64, 128])),
        Bq=int(r.choice([64, 128])), Bk=int(r.choice([64, 128])), score=int(r.integers(0, 2)),
        rho=(int(r.integers(10, 61)), 100), force_diag=bool(r.integers(0, 2)),
        win_T=int(r.choice([-1, -1, 1, 2])), win_r0=int(r.integers(0, 4)),
        orders=r.integers(0, 6, 3).astype(np.uint8), seed=5200 + k)


@pytest.mark.parametrize("k", range(NCASES))
def test_random_shape(bsa_gpu, orc, k):
    c = _draw(k)
    F, H, W, N, G, d = c["F"], c["H"], c["W"], c["N"], c["G"], c["d"]
    Bq, Bk = c["Bq"], c["Bk"]
    orders = c["orders"][:G].copy()
    _say(f"[random shape {k}] F={F} H={H} W={W} N={N} G={G} d={d} {Bq}x{Bk} score={c['score']} "
         f"rho={c['rho']} diag={c['force_diag']} win=({c['win_T']},{c['win_r0']}) orders={orders.tolist()}")
    r = np.random.Generator(np.random.PCG64(c["seed"]))
    nat = [r.standard_normal((N, G, d)).astype(np.float32) for _ in range(3)]
    dev = [_bf16(x) for x in nat]
    od = torch.from_numpy(orders).cuda()
    Qp, Kp, Vp = (bsa_gpu.permute(x, od, F, H, W, 0) for x in dev)

    # mask build, bit for bit
    p = bsa_gpu.mask_params(Bq, Bk, c["score"], c["rho"], c["force_diag"], c["win_T"], c["win_r0"])
    grp, gci, gnnz = bsa_gpu.build_mask(Qp, Kp, od, F, H, W, p)
    torch.cuda.synchronize()
    host = [orc.f32_to_bf16(x) for x in nat]  # the same bf16 values, converted by the oracle
    host_p = [orc.permute(0, h, np.uint16, G, F, H, W, d, orders) for h in host]
    wrp, wci = orc.build_mask(host_p[0], host_p[1], F, H, W, orders, Bq, Bk, c["score"], c["rho"][0],
                              c["rho"][1], int(c["force_diag"]), c["win_T"], c["win_r0"])
    n = int(_np(gnnz)[0])
    assert n == int(wrp[-1])
    assert np.array_equal(_np(grp), wrp)
    assert np.array_equal(_np(gci)[:n], wci)

    # bf16 forward, natural-order output, every row
    O, lse = bsa_gpu.forward_natural(Qp, Kp, Vp, grp, gci, Bq, Bk, od, F, H, W)
    torch.cuda.synchronize()
    rows = np.array([(g, t) for g in range(G) for t in range(N)], np.int64)
    Ow, Lw = orc.attention_rows(*host, G, F, H, W, d, orders, rows, Bq, Bk, wrp, wci)
    _compare(_np(O.float())[rows[:, 1], rows[:, 0]], Ow, f"bf16 case {k}", heads=rows[:, 0])
    lg = _np(lse)[rows[:, 0], rows[:, 1]]
    fin = np.isfinite(Lw)
    assert np.array_equal(fin, np.isfinite(lg))
    assert np.all(np.abs(lg[fin] - Lw[fin]) <= LSE_ABS)

    # first-order compensation of the skipped keys, on the same output
    bsa_gpu.fo_compensate(Qp, Kp, Vp, grp, gci, Bq, Bk, O, lse, od, F, H, W)
    torch.cuda.synchronize()
    half = rows[::2]
    Oc, Lc = orc.attention_rows_fo(*host, G, F, H, W, d, orders, half, Bq, Bk, wrp, wci)
    _compare(_np(O.float())[half[:, 1], half[:, 0]], Oc, f"compensated case {k}", heads=half[:, 0])
    lg = _np(lse)[half[:, 0], half[:, 1]]
    fin = np.isfinite(Lc)
    assert np.array_equal(fin, np.isfinite(lg))
    assert np.all(np.abs(lg[fin] - Lc[fin]) <= LSE_ABS + 2.0 ** -21 * np.abs(Lc[fin]))

    # INT8 forward on the same mask
    _int8_all_blocks(bsa_gpu, orc, Qp, Kp, Vp, wrp, wci, Bq, Bk, f"int8 case {k}", host_p)


@pytest.mark.parametrize("k", range(NCASES))
def test_random_shape_order_choice_and_calibration(bsa_gpu, orc, k):
    """The same draws through the order choice and the offline calibration:
    SICS scores of Q and K over the six axis orders bit for bit and the same
    chosen orders; block statistics of the dense map (block = Bq) with each
    count inside the oracle's bracket at eps(1 -+ 1e-3) and equal where no
    entry lies in it, sums and maxima within 2e-4 relative."""
    c = _draw(k)
    F, H, W, N, G, d, B = c["F"], c["H"], c["W"], c["N"], c["G"], c["d"], c["Bq"]
    orders = c["orders"][:G].copy()
    _say(f"[random shape {k}: order choice and calibration] N={N} G={G} d={d} B={B}")
    r = np.random.Generator(np.random.PCG64(c["seed"]))
    nat = [r.standard_normal((N, G, d)).astype(np.float32) for _ in range(3)]
    dev = [_bf16(x) for x in nat[:2]]
    host = [orc.f32_to_bf16(x) for x in nat[:2]]

    sq = bsa_gpu.order_scores(dev[0], F, H, W, B)
    sk = bsa_gpu.order_scores(dev[1], F, H, W, B)
    chosen = bsa_gpu.select_orders(sq, sk)
    torch.cuda.synchronize()
    wq = orc.sics_scores(host[0], G, F, H, W, d, B)
    wk = orc.sics_scores(host[1], G, F, H, W, d, B)
    assert np.array_equal(_np(sq).view(np.uint32), wq.view(np.uint32))
    assert np.array_equal(_np(sk).view(np.uint32), wk.view(np.uint32))
    assert np.array_equal(_np(chosen), orc.select_orders(wq, wk))

    od = torch.from_numpy(orders).cuda()
    Qp, Kp = (bsa_gpu.permute(x, od, F, H, W, 0) for x in dev)
    cnt, bsum, bmax = bsa_gpu.attn_block_stats(Qp, Kp, B, 1e-3)
    torch.cuda.synchronize()
    host_p = [orc.permute(0, h, np.uint16, G, F, H, W, d, orders) for h in host]
    want = orc.block_stats(host_p[0], host_p[1], B, 1e-3, delta=1e-3)
    cn = _np(cnt)
    assert np.all(want["cnt_lo"] <= cn) and np.all(cn <= want["cnt_hi"])
    sure = want["cnt_lo"] == want["cnt_hi"]
    assert np.array_equal(cn[sure], want["cnt"][sure])
    assert np.allclose(_np(bsum).astype(np.float64), want["sum"], rtol=2e-4, atol=1e-9)
    assert np.allclose(_np(bmax).astype(np.float64), want["max"], rtol=2e-4, atol=1e-12)
