"""GPU parity of the first-order compensation of the skipped keys
(bsa_fo_compensate after bsa_forward / bsa_forward_natural) against the
CPU oracle's masked attention with the same compensation, on the same
seeded inputs: relative L2 <= 1e-2 and max |diff| <= 2e-2 on O, lse within
1e-3 (plus a few fp32 ulps of its magnitude)."""
import numpy as np
import pytest
import torch

from test_gpu_parity import _bits, _compare, _np, _say, case, oracle_reorder, mask_params, sample_rows

pytestmark = pytest.mark.gpu

LSE_ABS = 1e-3


def _static(cfg, seed):
    from block_sparse_attention_inverse_amd import synth

    return synth.static_mask(cfg["G"], cfg["N"], cfg["Bq"], cfg["Bk"], cfg["k_static"], seed)


def _gpu_chain(bsa, c, rp, ci, Bq, Bk, natural=True):
    cfg = c["cfg"]
    F, H, W = cfg["F"], cfg["H"], cfg["W"]
    Qp, Kp, Vp = (bsa.permute(c[x], c["orders_dev"], F, H, W, 0) for x in ("Q", "K", "V"))
    grp, gci = (torch.from_numpy(x).cuda() if isinstance(x, np.ndarray) else x for x in (rp, ci))
    if natural:
        O, lse = bsa.forward_natural(Qp, Kp, Vp, grp, gci, Bq, Bk, c["orders_dev"], F, H, W)
        bsa.fo_compensate(Qp, Kp, Vp, grp, gci, Bq, Bk, O, lse, c["orders_dev"], F, H, W)
    else:
        O, lse = bsa.forward(Qp, Kp, Vp, grp, gci, Bq, Bk)
        bsa.fo_compensate(Qp, Kp, Vp, grp, gci, Bq, Bk, O, lse, F=F, H=H, W=W)
    torch.cuda.synchronize()
    return O, lse


def _check_rows(orc, c, O, lse, rows, rp, ci, Bq, Bk, natural, tag):
    cfg = c["cfg"]
    G, F, H, W, d, N = cfg["G"], cfg["F"], cfg["H"], cfg["W"], cfg["d"], cfg["N"]
    src = c["host"]
    Ow, Lw = orc.attention_rows_fo(src["Q"], src["K"], src["V"], G, F, H, W, d, c["orders"], rows, Bq,
                                   Bk, rp, ci)
    On, Ln = _np(O.float()), _np(lse)
    if natural:
        got = On[rows[:, 1], rows[:, 0]]
        lg = Ln[rows[:, 0], rows[:, 1]]
    else:
        pos = {}
        for g in np.unique(rows[:, 0]):
            pm = orc.perm(int(c["orders"][g]), F, H, W)
            inv = np.empty(N, np.int64)
            inv[pm] = np.arange(N)
            pos[g] = inv
        p = np.array([pos[g][n] for g, n in rows])
        got = On[rows[:, 0], p]
        lg = Ln[rows[:, 0], p]
    _compare(got, Ow, heads=rows[:, 0], tag=tag)
    tol = LSE_ABS + 2.0 ** -21 * np.abs(Lw)
    err = np.abs(lg - Lw)
    _say(f"  lse max_abs={err.max():.3e}")
    assert np.all(err <= tol)


@pytest.mark.parametrize("natural", [True, False])
def test_compensation_2k_static(bsa_gpu, orc, natural):
    """2k layer (8 heads, d=64, 64x64 blocks, static 31 % mask): every third
    row of every head, natural-order and reordered outputs."""
    c = case(2)
    cfg = c["cfg"]
    rp, ci = _static(cfg, c["seed"])
    _say(f"[compensation 2k natural={natural}]")
    O, lse = _gpu_chain(bsa_gpu, c, rp, ci, cfg["Bq"], cfg["Bk"], natural)
    rows = np.array([(g, n) for g in range(cfg["G"]) for n in range(0, cfg["N"], 3)], np.int64)
    _check_rows(orc, c, O, lse, rows, rp, ci, cfg["Bq"], cfg["Bk"], natural, f"fo cfg2 nat={natural}")


def test_compensation_480p_built_mask(bsa_gpu, orc):
    """480p layer (12 heads, d=128, 128x64 blocks, DOT top-k 30 %): the mask
    built on the GPU, rows sampled from the first, the last (ragged) and
    random q-blocks."""
    c = case(3)
    cfg = c["cfg"]
    F, H, W = cfg["F"], cfg["H"], cfg["W"]
    p = mask_params(bsa_gpu, cfg)
    Qp, Kp, _ = (bsa_gpu.permute(c[x], c["orders_dev"], F, H, W, 0) for x in ("Q", "K", "V"))
    grp, gci, gnnz = bsa_gpu.build_mask(Qp, Kp, c["orders_dev"], F, H, W, p)
    rp, ci = orc.build_mask(oracle_reorder(orc, c, "Q"), oracle_reorder(orc, c, "K"), F, H, W,
                            c["orders"], p.Bq, p.Bk, p.score, p.rho_num, p.rho_den, p.force_diag,
                            p.win_T, p.win_r0)
    assert int(_np(gnnz)[0]) == len(ci)
    _say("[compensation 480p]")
    O, lse = _gpu_chain(bsa_gpu, c, grp, gci, p.Bq, p.Bk, True)
    rows = sample_rows(cfg, c["orders"], orc, 24, c["seed"] + 21)
    _check_rows(orc, c, O, lse, rows, rp, ci, p.Bq, p.Bk, True, "fo cfg3")


@pytest.mark.parametrize("d,Bq,Bk", [(128, 128, 128), (64, 128, 64), (128, 64, 128)])
def test_compensation_shapes_and_ragged_tail(bsa_gpu, orc, d, Bq, Bk):
    """Other head dims and block shapes on a ragged grid (N = 424): every row
    against the oracle, natural-order output."""
    from block_sparse_attention_inverse_amd import synth

    F, H, W, G = 2, 4, 53, 2
    N = F * H * W
    r = np.random.Generator(np.random.PCG64(900 + d + Bq + Bk))
    orders = np.array([5, 2], np.uint8)
    nat = [torch.from_numpy(r.standard_normal((N, G, d)).astype(np.float32)).to(torch.bfloat16).cuda()
           for _ in range(3)]
    nk = -(-N // Bk)
    rp, ci = synth.static_mask(G, N, Bq, Bk, max(1, nk // 3), 950 + d)
    cfg = dict(G=G, F=F, H=H, W=W, d=d, N=N, Bq=Bq, Bk=Bk)
    c = dict(cfg=cfg, orders=orders, orders_dev=torch.from_numpy(orders).cuda(),
             Q=nat[0], K=nat[1], V=nat[2], host={k: _bits(x) for k, x in zip("QKV", nat)})
    _say(f"[compensation d={d} {Bq}x{Bk}]")
    O, lse = _gpu_chain(bsa_gpu, c, rp, ci, Bq, Bk, True)
    rows = np.array([(g, n) for g in range(G) for n in range(N)], np.int64)
    _check_rows(orc, c, O, lse, rows, rp, ci, Bq, Bk, True, f"fo d={d} {Bq}x{Bk}")


def test_compensation_reaches_dense_attention_when_skipped_keys_agree(bsa_gpu):
    """Every skipped key is the same vector: the first-order compensation is
    then exact and the compensated block-sparse output equals dense attention
    (fp64 on the CPU) up to the bf16 rounding of inputs, moments and output."""
    r = np.random.Generator(np.random.PCG64(77))
    F, H, W, G, d, B = 1, 4, 64, 2, 128, 64
    N = F * H * W
    Q = r.standard_normal((N, G, d)).astype(np.float32)
    V = r.standard_normal((N, G, d)).astype(np.float32)
    K = np.repeat(r.standard_normal((1, G, d)).astype(np.float32), N, axis=0)
    K[:B] = r.standard_normal((B, G, d))  # block 0 (identity order): free keys, kept by every row
    nb = N // B
    sets = [[0] if i == 0 else [0, i] for _ in range(G) for i in range(nb)]
    rp = np.cumsum([0] + [len(x) for x in sets]).astype(np.int32)
    ci = np.array([j for x in sets for j in x], np.int32)
    import block_sparse_attention_inverse_amd as bsa

    od = torch.zeros(G, dtype=torch.uint8).cuda()
    dev = [torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (Q, K, V)]
    Qp, Kp, Vp = (bsa.permute(x, od, F, H, W, 0) for x in dev)
    grp, gci = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    O, lse = bsa.forward_natural(Qp, Kp, Vp, grp, gci, B, B, od, F, H, W)
    O0 = O.float().clone()
    bsa.fo_compensate(Qp, Kp, Vp, grp, gci, B, B, O, lse, od, F, H, W)
    torch.cuda.synchronize()
    q, k, v = (x.cpu().double() for x in dev)  # the bf16 inputs, exactly
    s = torch.einsum("ngc,mgc->gnm", q, k) / np.sqrt(d)
    ref = torch.einsum("gnm,mgc->ngc", torch.softmax(s, dim=-1), v).numpy()
    got = O.float().cpu().numpy()
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    err0 = np.linalg.norm(O0.cpu().numpy() - ref) / np.linalg.norm(ref)
    _say(f"  compensated rel_l2 vs dense {err:.3e} (masked only {err0:.3e})")
    assert err < 1e-2 and err0 > 5e-2


def test_compensation_shared_mask_strided_output_and_scale(bsa_gpu, orc):
    """Batch copies sharing one mask (mask_G = 2 of G = 4 heads), the
    natural-order output written into a strided [G][N][d] buffer viewed as
    [N][G][d], and an explicit softmax scale: every row against the oracle."""
    from block_sparse_attention_inverse_amd import synth

    F, H, W, G, d, B = 2, 6, 21, 4, 64, 64
    N = F * H * W
    mask_G = 2
    sm = 0.21
    r = np.random.Generator(np.random.PCG64(4242))
    orders = np.array([3, 1, 4, 0], np.uint8)
    nat = [torch.from_numpy(r.standard_normal((N, G, d)).astype(np.float32)).to(torch.bfloat16).cuda()
           for _ in range(3)]
    rp, ci = synth.static_mask(mask_G, N, B, B, 2, 4343)
    od = torch.from_numpy(orders).cuda()
    Qp, Kp, Vp = (bsa_gpu.permute(x, od, F, H, W, 0) for x in nat)
    grp, gci = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    base = torch.full((G, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    Ov = base.transpose(0, 1)  # [N][G][d] view, strides (d, N*d, 1)
    _, lse = bsa_gpu.forward_natural(Qp, Kp, Vp, grp, gci, B, B, od, F, H, W, mask_G=mask_G,
                                     sm_scale=sm, out=Ov)
    bsa_gpu.fo_compensate(Qp, Kp, Vp, grp, gci, B, B, Ov, lse, od, F, H, W, mask_G=mask_G,
                          sm_scale=sm)
    torch.cuda.synchronize()
    _say("[compensation shared mask, strided output, sm_scale 0.21]")
    host = {k: _bits(x) for k, x in zip("QKV", nat)}
    rows = np.array([(g, n) for g in range(G) for n in range(N)], np.int64)
    Ow, Lw = orc.attention_rows_fo(host["Q"], host["K"], host["V"], G, F, H, W, d, orders, rows, B, B,
                                   rp, ci, mask_G=mask_G, sm_scale=sm)
    got = _np(Ov.float())[rows[:, 1], rows[:, 0]]
    _compare(got, Ow, heads=rows[:, 0], tag="fo shared mask strided")
    lg = _np(lse)[rows[:, 0], rows[:, 1]]
    err = np.abs(lg - Lw)
    _say(f"  lse max_abs={err.max():.3e}")
    assert np.all(err <= LSE_ABS + 2.0 ** -21 * np.abs(Lw))


def test_compensation_leaves_rows_without_skipped_keys_unchanged(bsa_gpu, orc):
    """Every kv-block kept (100 % density, nothing skipped): O and lse come
    back bit for bit; with one row of q-blocks empty instead (nothing kept),
    that row's output becomes the compensation alone, finite and equal to the
    oracle's."""
    F, H, W, G, d, B = 1, 5, 40, 2, 128, 64
    N = F * H * W
    nq = nk = -(-N // B)
    r = np.random.Generator(np.random.PCG64(515))
    od = torch.zeros(G, dtype=torch.uint8).cuda()
    nat = [torch.from_numpy(r.standard_normal((N, G, d)).astype(np.float32)).to(torch.bfloat16).cuda()
           for _ in range(3)]
    Qp, Kp, Vp = (bsa_gpu.permute(x, od, F, H, W, 0) for x in nat)
    rp = np.arange(0, G * nq * nk + 1, nk, dtype=np.int32)
    ci = np.tile(np.arange(nk, dtype=np.int32), G * nq)
    grp, gci = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    O, lse = bsa_gpu.forward_natural(Qp, Kp, Vp, grp, gci, B, B, od, F, H, W)
    O0, L0 = O.clone(), lse.clone()
    bsa_gpu.fo_compensate(Qp, Kp, Vp, grp, gci, B, B, O, lse, od, F, H, W)
    torch.cuda.synchronize()
    _say("[compensation, nothing skipped]")
    assert torch.equal(O.view(torch.int16), O0.view(torch.int16))
    assert torch.equal(lse, L0)
    # q-block 0 of every head keeps nothing: its rows get the compensation alone
    sets = [[] if i == 0 else list(range(nk)) for _ in range(G) for i in range(nq)]
    rp2 = np.cumsum([0] + [len(x) for x in sets]).astype(np.int32)
    ci2 = np.array([j for x in sets for j in x], np.int32)
    grp2, gci2 = torch.from_numpy(rp2).cuda(), torch.from_numpy(ci2).cuda()
    O2, l2 = bsa_gpu.forward_natural(Qp, Kp, Vp, grp2, gci2, B, B, od, F, H, W)
    torch.cuda.synchronize()
    assert torch.all(O2[:B].float() == 0) and torch.all(torch.isinf(l2[:, :B]))
    bsa_gpu.fo_compensate(Qp, Kp, Vp, grp2, gci2, B, B, O2, l2, od, F, H, W)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(O2.float())) and torch.all(torch.isfinite(l2))
    assert float(O2[:B].float().abs().sum()) > 0
    host = {k: _bits(x) for k, x in zip("QKV", nat)}
    rows = np.array([(g, n) for g in range(G) for n in range(B)], np.int64)
    Ow, Lw = orc.attention_rows_fo(host["Q"], host["K"], host["V"], G, F, H, W, d,
                                   np.zeros(G, np.uint8), rows, B, B, rp2, ci2)
    got = _np(O2.float())[rows[:, 1], rows[:, 0]]
    _compare(got, Ow, heads=rows[:, 0], tag="fo empty rows")
    err = np.abs(_np(l2)[rows[:, 0], rows[:, 1]] - Lw)
    _say(f"  lse max_abs={err.max():.3e}")
    assert np.all(err <= LSE_ABS + 2.0 ** -21 * np.abs(Lw))


@pytest.mark.parametrize("int8,fused", [(False, True), (True, True), (False, False)])
def test_layer_forward_with_compensation(bsa_gpu, int8, fused):
    """layer_forward with compensate=True gives, bit for bit, the same chain
    without it followed by bsa_fo_compensate on its output (480p layer, mask
    built from the sums or from Qp and Kp)."""
    c = case(3)
    cfg = c["cfg"]
    G, F, H, W, d = cfg["G"], cfg["F"], cfg["H"], cfg["W"], cfg["d"]
    p = mask_params(bsa_gpu, cfg)
    od = c["orders_dev"]
    _say(f"[layer_forward compensate int8={int8} fused={fused}]")
    plan = bsa_gpu.LayerPlan(G, F, H, W, d, "cuda", p, int8=int8, fused=fused, compensate=True)
    got = bsa_gpu.layer_forward(plan, c["Q"], c["K"], c["V"], od).clone()
    got_lse = plan.lse.clone()
    ref = bsa_gpu.LayerPlan(G, F, H, W, d, "cuda", p, int8=int8, fused=fused)
    out = bsa_gpu.layer_forward(ref, c["Q"], c["K"], c["V"], od)
    # the bf16 reordered inputs the compensation reads (the INT8 chain skips them)
    Qp, Kp, Vp = (bsa_gpu.permute(c[x], od, F, H, W, 0) for x in ("Q", "K", "V"))
    if fused:
        bsa_gpu.fo_compensate(Qp, Kp, Vp, ref.row_ptr, ref.col_idx, p.Bq, p.Bk, out, ref.lse, od,
                              F, H, W)
    else:
        bsa_gpu.fo_compensate(Qp, Kp, Vp, ref.row_ptr, ref.col_idx, p.Bq, p.Bk, ref.Op, ref.lse,
                              F=F, H=H, W=W)
        out = bsa_gpu.permute(ref.Op, od, F, H, W, 1)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), out.view(torch.int16))
    assert torch.equal(got_lse, ref.lse)
