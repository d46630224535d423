"""GPU parity of the selection from a score matrix: the block scores, Top-K
(with and without seeded noise perturbing the scores) and Top-P, through the
C ABI against the CPU oracle on the same seeded inputs.

Bars: scores, Top-K and Top-P CSRs are outputs of fixed fp32 sequences and
match bit for bit.  Top-P weighs the sorted scores with a fixed fp32 2^x
(range reduction to the nearest integer, a degree-7 Taylor polynomial by
fma, an exact power-of-two scale) that the kernel and the oracle each
implement, and adds the weights in sorted order on both sides.
"""
import numpy as np
import pytest
import torch

from test_gpu_parity import _np, _say, case, mask_params, oracle_reorder

pytestmark = pytest.mark.gpu


def _sums(bsa, c, p):
    cfg = c["cfg"]
    F, H, W = cfg["F"], cfg["H"], cfg["W"]
    _, sq, _ = bsa.permute_pool(c["Q"], c["orders_dev"], F, H, W, p.Bq, sums=True, reordered=False)
    _, sk, _ = bsa.permute_pool(c["K"], c["orders_dev"], F, H, W, p.Bk, sums=True, reordered=False)
    return sq, sk


def _oracle_keys(orc, c, p):
    """The oracle's block keys from the host inputs: its own reorder, block
    sums and keys (nothing taken from the GPU)."""
    cfg = c["cfg"]
    G, N = cfg["G"], cfg["F"] * cfg["H"] * cfg["W"]
    sq = orc.block_sums(oracle_reorder(orc, c, "Q"), p.Bq)
    sk = orc.block_sums(oracle_reorder(orc, c, "K"), p.Bk)
    return np.stack([orc.block_keys(sq[g], sk[g], N, p.Bq, p.Bk, p.score) for g in range(G)])


SCORE_CASES = [
    # (cid, overrides, rho)
    (2, {}, None),
    (2, dict(mask="cosine", rho=(25, 100), win_T=1, win_r0=2, Bq=64, Bk=64), None),
    (3, {}, None),
    (5, {}, None),
]


@pytest.mark.parametrize("cid,over,rho", SCORE_CASES)
def test_block_scores_and_topk_bit_exact(bsa_gpu, orc, cid, over, rho):
    """bsa_block_scores equals the oracle's keys bit for bit, and Top-K on
    them equals bsa_build_mask_pooled and the oracle's selection."""
    c = case(cid)
    cfg = dict(c["cfg"], **over)
    G, F, H, W = cfg["G"], cfg["F"], cfg["H"], cfg["W"]
    p = mask_params(bsa_gpu, cfg, rho)
    _say(f"[scores cfg {cid} {over}] score={p.score} win={p.win_T}")
    sq, sk = _sums(bsa_gpu, c, p)
    sc = bsa_gpu.block_scores(sq, sk, F, H, W, p)
    rp, ci, nnz = bsa_gpu.mask_from_scores(sc, c["orders_dev"], F, H, W, p)
    rp2, ci2, nnz2 = bsa_gpu.build_mask_pooled(sq, sk, c["orders_dev"], F, H, W, p)
    torch.cuda.synchronize()
    want = _oracle_keys(orc, c, p)
    assert np.array_equal(_np(sc).view(np.uint32), want.view(np.uint32))
    n = int(_np(nnz)[0])
    assert n == int(_np(nnz2)[0])
    assert np.array_equal(_np(rp), _np(rp2)) and np.array_equal(_np(ci)[:n], _np(ci2)[:n])
    wrp, wci = orc.select(want, G, F, H, W, p.Bq, p.Bk, c["orders"], p.rho_num, p.rho_den,
                          p.force_diag, p.win_T, p.win_r0)
    assert np.array_equal(_np(rp), wrp) and np.array_equal(_np(ci)[:n], wci)


@pytest.mark.parametrize("cid,scale", [(2, 0.5), (3, 2.0), (5, 0.05)])
def test_topk_with_noise_bit_exact(bsa_gpu, orc, cid, scale):
    """Scores perturbed by seeded Gumbel noise (the stochastic scoring):
    key' = fmaf(noise, scale, key), then Top-K and the forced set."""
    c = case(cid)
    cfg = c["cfg"]
    G, F, H, W = cfg["G"], cfg["F"], cfg["H"], cfg["W"]
    p = mask_params(bsa_gpu, cfg)
    sq, sk = _sums(bsa_gpu, c, p)
    sc = bsa_gpu.block_scores(sq, sk, F, H, W, p)
    r = np.random.Generator(np.random.PCG64(500 + cid))
    noise = r.gumbel(size=tuple(sc.shape)).astype(np.float32)
    _say(f"[noisy top-k cfg {cid} scale {scale}]")
    rp, ci, nnz = bsa_gpu.mask_from_scores(sc, c["orders_dev"], F, H, W, p,
                                           noise=torch.from_numpy(noise).cuda(), noise_scale=scale)
    torch.cuda.synchronize()
    want = _oracle_keys(orc, c, p)
    assert np.array_equal(_np(sc).view(np.uint32), want.view(np.uint32))
    kp = orc.perturb_keys(want, noise, scale)
    wrp, wci = orc.select(kp, G, F, H, W, p.Bq, p.Bk, c["orders"], p.rho_num, p.rho_den,
                          p.force_diag, p.win_T, p.win_r0)
    n = int(_np(nnz)[0])
    assert np.array_equal(_np(rp), wrp) and np.array_equal(_np(ci)[:n], wci)
    # the noise does move the selection
    rp0, ci0, n0 = bsa_gpu.mask_from_scores(sc, c["orders_dev"], F, H, W, p)
    torch.cuda.synchronize()
    assert not np.array_equal(_np(ci0)[:int(_np(n0)[0])], wci)


def _topp_compare(orc, got_rp, got_ci, keys, G, F, H, W, p, orders, top_p, temp, noise=None,
                  scale=0.0):
    """Top-P CSR bit for bit: both sides weigh the sorted scores with the same
    fixed fp32 2^x sequence and add the weights in the same order."""
    kp = keys if noise is None else orc.perturb_keys(keys, noise, scale)
    wrp, wci, kstar, cum = orc.select_topp(kp, G, F, H, W, p.Bq, p.Bk, orders, top_p, temp,
                                           p.force_diag, p.win_T, p.win_r0)
    assert np.array_equal(got_rp, wrp)
    assert np.array_equal(got_ci, wci)
    return wrp, wci


@pytest.mark.parametrize("cid,top_p,temp", [(2, 0.9, 1.0), (2, 0.99, 16.0), (3, 0.5, 4.0),
                                            (3, 0.95, 0.25), (5, 0.8, 8.0), (5, 0.3, 0.5),
                                            (4, 0.9, 2.0)])
def test_topp_parity(bsa_gpu, orc, cid, top_p, temp):
    c = case(cid)
    cfg = c["cfg"]
    G, F, H, W = cfg["G"], cfg["F"], cfg["H"], cfg["W"]
    p = mask_params(bsa_gpu, cfg)
    sq, sk = _sums(bsa_gpu, c, p)
    sc = bsa_gpu.block_scores(sq, sk, F, H, W, p)
    _say(f"[top-p cfg {cid} p={top_p} temp={temp}]")
    rp, ci, nnz = bsa_gpu.mask_from_scores(sc, c["orders_dev"], F, H, W, p, top_p=top_p, temp=temp)
    torch.cuda.synchronize()
    n = int(_np(nnz)[0])
    want = _oracle_keys(orc, c, p)
    assert np.array_equal(_np(sc).view(np.uint32), want.view(np.uint32))
    _topp_compare(orc, _np(rp), _np(ci)[:n], want, G, F, H, W, p, c["orders"], top_p, temp)


def test_topp_with_noise_and_exact_weights(bsa_gpu, orc):
    """Integer scores at temp 1 (every weight a power of two, every sum
    exact) with integer-valued noise: the cut is exact on both sides, so the
    CSR matches bit for bit; temp 0 (uniform weights) likewise."""
    cfg = case(2)["cfg"]
    G, F, H, W = cfg["G"], cfg["F"], cfg["H"], cfg["W"]
    c = case(2)
    p = mask_params(bsa_gpu, cfg)
    N = F * H * W
    nq, nk = -(-N // p.Bq), -(-N // p.Bk)
    r = np.random.Generator(np.random.PCG64(77))
    keys = r.integers(-12, 1, size=(G, nq, nk)).astype(np.float32)
    noise = r.integers(-2, 3, size=(G, nq, nk)).astype(np.float32)
    for top_p, temp, nz in ((0.75, 1.0, None), (0.6, 1.0, noise), (0.5, 0.0, None), (1.0, 1.0, noise)):
        _say(f"[top-p exact p={top_p} temp={temp} noise={nz is not None}]")
        rp, ci, nnz = bsa_gpu.mask_from_scores(
            torch.from_numpy(keys).cuda(), c["orders_dev"], F, H, W, p, top_p=top_p, temp=temp,
            noise=None if nz is None else torch.from_numpy(nz).cuda(), noise_scale=1.0)
        torch.cuda.synchronize()
        kp = keys if nz is None else orc.perturb_keys(keys, nz, 1.0)
        wrp, wci, _, _ = orc.select_topp(kp, G, F, H, W, p.Bq, p.Bk, c["orders"], top_p, temp,
                                         p.force_diag, p.win_T, p.win_r0)
        n = int(_np(nnz)[0])
        assert np.array_equal(_np(rp), wrp) and np.array_equal(_np(ci)[:n], wci)
