"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on
the same seeded synthetic inputs.

Bit-exact: reordering, CSR (row_ptr, col_idx, nnz), INT8 codes and scales,
integer tile products.  Floating point (bf16 and INT8 attention outputs,
natural order): relative L2 <= 1e-2 and max |diff| <= 2e-2, over the whole
compared set and per head; LSE within 1e-3 (diagnostic).
"""
import functools

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_ABS = 2e-2
LSE_ABS = 1e-3
# fp32 inputs are rounded to bf16 by the reordering while the oracle attends
# on the fp32 values: each score moves by up to sm_scale*sum|q k|*2^-8
# (two operands, half-ulp 2^-9 each), a few 1e-3 at d=64; LSE moves as much.
LSE_ABS_F32_INPUT = 1e-2


def _say(msg):
    print(msg, flush=True)


def _np(t):
    return t.detach().cpu().numpy()


def _bits(t):
    from block_sparse_attention_inverse_amd import synth

    return synth.bf16_bits(t)


def _f64_from_bits(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _compare(got, want, heads=None, tag=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    diff = got - want
    rel = np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-30)
    mx = np.max(np.abs(diff)) if diff.size else 0.0
    _say(f"  {tag}: rel_l2={rel:.3e} max_abs={mx:.3e} n={diff.shape[0]}")
    assert rel <= REL_L2, f"{tag}: rel L2 {rel}"
    assert mx <= MAX_ABS, f"{tag}: max abs {mx}"
    if heads is not None:
        for g in np.unique(heads):
            sel = heads == g
            rg = np.linalg.norm(diff[sel]) / max(np.linalg.norm(want[sel]), 1e-30)
            assert rg <= REL_L2, f"{tag}: head {g} rel L2 {rg}"


# ------------------------------------------------------------------ cases
@functools.lru_cache(maxsize=2)
def case(cid, **over):
    """Seeded inputs of configuration ``cid`` on the GPU plus host copies."""
    from block_sparse_attention_inverse_amd import synth

    cfg = synth.config(cid, **over)
    seed = synth.seed_of(cid)
    orders = synth.make_orders(cfg, seed)
    _say(f"[case {cid}] generating N={cfg['N']} G={cfg['G']} d={cfg['d']} seed={seed}")
    Q, K, V = synth.cast_inputs(cfg, *synth.make_qkv(cfg, orders, seed, device="cuda"))
    torch.cuda.synchronize()
    host = {}
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        host[name] = _bits(t) if t.dtype == torch.bfloat16 else _np(t)
    return dict(cfg=cfg, seed=seed, orders=orders, Q=Q, K=K, V=V, host=host,
                orders_dev=torch.from_numpy(orders).cuda())


def gpu_reorder(bsa, c):
    cfg = c["cfg"]
    F, H, W = cfg["F"], cfg["H"], cfg["W"]
    return [bsa.permute(c[x], c["orders_dev"], F, H, W, 0) for x in ("Q", "K", "V")]


def oracle_reorder(orc, c, name):
    cfg = c["cfg"]
    src = c["host"][name]
    return orc.permute(0, src, np.uint16, cfg["G"], cfg["F"], cfg["H"], cfg["W"], cfg["d"],
                       c["orders"])


def mask_params(bsa, cfg, rho=None):
    if cfg["mask"] == "cosine":
        return bsa.mask_params(cfg["Bq"], cfg["Bk"], 1, rho or cfg["rho"], True, cfg["win_T"],
                               cfg["win_r0"])
    return bsa.mask_params(cfg["Bq"], cfg["Bk"], 0, rho or cfg.get("rho", (30, 100)), True)


def sample_rows(cfg, orders, orc, n_rand, seed):
    """(g, n) natural rows: random ones plus, per head, rows whose reordered
    position lies in the first and in the last (ragged) q-block."""
    r = np.random.Generator(np.random.PCG64(seed))
    G, N, Bq = cfg["G"], cfg["N"], cfg["Bq"]
    rows = [(int(r.integers(G)), int(r.integers(N))) for _ in range(n_rand)]
    last0 = ((N - 1) // Bq) * Bq
    for g in range(G):
        pm = orc.perm(int(orders[g]), cfg["F"], cfg["H"], cfg["W"])
        for p in (0, Bq - 1, last0, N - 1):
            rows.append((g, int(pm[p])))
    return np.array(rows, np.int64)


# ------------------------------------------------------------ reordering
@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_permute_bit_exact(bsa_gpu, orc, cid):
    c = case(cid)
    cfg = c["cfg"]
    G, F, H, W, d = cfg["G"], cfg["F"], cfg["H"], cfg["W"], cfg["d"]
    _say(f"[permute cfg {cid}]")
    Qp = bsa_gpu.permute(c["Q"], c["orders_dev"], F, H, W, 0)
    torch.cuda.synchronize()
    src = c["host"]["Q"]
    want = orc.permute(0, src, np.uint16, G, F, H, W, d, c["orders"])
    assert np.array_equal(_bits(Qp), want)
    # inverse: reordered -> natural, into fp32 and into bf16
    back = bsa_gpu.permute(Qp, c["orders_dev"], F, H, W, 1)
    back32 = bsa_gpu.permute(Qp, c["orders_dev"], F, H, W, 1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    nat = orc.permute(1, want, np.uint16, G, F, H, W, d, c["orders"])
    assert np.array_equal(_bits(back), nat)
    assert np.array_equal(_np(back32), _f64_from_bits(nat).astype(np.float32))
    if cfg["dtype"] != "f32":
        assert np.array_equal(_bits(back), src)


def test_permute_strided_natural_layouts(bsa_gpu, orc):
    """[G][N][d] natural layout (as a strided view) and a strided output."""
    c = case(2)
    cfg = c["cfg"]
    G, F, H, W, d, N = cfg["G"], cfg["F"], cfg["H"], cfg["W"], cfg["d"], cfg["N"]
    xg = c["K"].transpose(0, 1).contiguous()  # [G][N][d]
    view = xg.transpose(0, 1)  # [N][G][d] view with stride_n = d, stride_g = N*d
    Kp = bsa_gpu.permute(view, c["orders_dev"], F, H, W, 0)
    out = torch.zeros((G, N, d), dtype=torch.bfloat16, device="cuda").transpose(0, 1)
    bsa_gpu.permute(Kp, c["orders_dev"], F, H, W, 1, out=out)
    torch.cuda.synchronize()
    want = oracle_reorder(orc, c, "K")
    assert np.array_equal(_bits(Kp), want)
    assert torch.equal(out.contiguous(), c["K"])


# ------------------------------------------------------------ mask build
MASK_CASES = [
    (2, dict(mask="dot", rho=(30, 100)), None),
    (2, dict(mask="cosine", rho=(25, 100), win_T=1, win_r0=2, Bq=64, Bk=64), None),
    (3, {}, None),
    (4, {}, None),
    (4, {}, (20, 100)),
    (5, {}, None),
]


@pytest.mark.parametrize("cid,over,rho", MASK_CASES)
def test_build_mask_bit_exact(bsa_gpu, orc, cid, over, rho):
    c = case(cid)
    cfg = dict(c["cfg"], **over)
    G, F, H, W = cfg["G"], cfg["F"], cfg["H"], cfg["W"]
    p = mask_params(bsa_gpu, cfg, rho)
    _say(f"[mask cfg {cid} {over} rho={rho}] Bq={p.Bq} Bk={p.Bk} score={p.score} win={p.win_T}")
    Qp, Kp, _ = gpu_reorder(bsa_gpu, c)
    rp, ci, nnz = bsa_gpu.build_mask(Qp, Kp, c["orders_dev"], F, H, W, p)
    torch.cuda.synchronize()
    oq, ok_ = oracle_reorder(orc, c, "Q"), oracle_reorder(orc, c, "K")
    wrp, wci, ties = orc.build_mask(oq, ok_, F, H, W, c["orders"], p.Bq, p.Bk, p.score,
                                    p.rho_num, p.rho_den, p.force_diag, p.win_T, p.win_r0,
                                    audit=True)
    n = int(_np(nnz)[0])
    _say(f"  nnz={n} rows={len(wrp) - 1} near_ties={ties}")
    assert n == int(wrp[-1])
    assert np.array_equal(_np(rp), wrp)
    assert np.array_equal(_np(ci)[:n], wci)


# ------------------------------------------------------------ quantize
@pytest.mark.parametrize("cid", [2, 3, 4])
def test_quantize_bit_exact(bsa_gpu, orc, cid):
    c = case(cid)
    cfg = c["cfg"]
    _say(f"[quantize cfg {cid}]")
    Qp, Kp, Vp = gpu_reorder(bsa_gpu, c)
    for name, x, B in (("Q", Qp, cfg["Bq"]), ("V", Vp, cfg["Bk"])):
        q, s = bsa_gpu.quantize_int8(x, B)
        torch.cuda.synchronize()
        wq, ws = orc.quantize_int8(oracle_reorder(orc, c, name), B)
        assert np.array_equal(_np(s), ws), name
        assert np.array_equal(_np(q), wq), name


# ------------------------------------------------------------ bf16 forward
def _static_csr(cfg, seed, dense=False):
    from block_sparse_attention_inverse_amd import synth

    if dense:
        return synth.dense_mask(cfg["G"], cfg["N"], cfg["Bq"], cfg["Bk"])
    return synth.static_mask(cfg["G"], cfg["N"], cfg["Bq"], cfg["Bk"], cfg["k_static"], seed)


def _run_forward_case(bsa, orc, c, rp, ci, rows, gpu_mask=None, tag=""):
    """GPU: reorder -> forward -> inverse; oracle: masked attention rows."""
    cfg = c["cfg"]
    G, F, H, W, d, N = cfg["G"], cfg["F"], cfg["H"], cfg["W"], cfg["d"], cfg["N"]
    Qp, Kp, Vp = gpu_reorder(bsa, c)
    if gpu_mask is None:
        grp, gci = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    else:
        grp, gci = gpu_mask
    Op, lse = bsa.forward(Qp, Kp, Vp, grp, gci, cfg["Bq"], cfg["Bk"])
    O = bsa.permute(Op, c["orders_dev"], F, H, W, 1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    On = _np(O)
    lse_h = _np(lse)
    src = c["host"]
    Ow, Lw = orc.attention_rows(src["Q"], src["K"], src["V"], G, F, H, W, d, c["orders"], rows,
                                cfg["Bq"], cfg["Bk"], rp, ci)
    got = On[rows[:, 1], rows[:, 0]]
    _compare(got, Ow, heads=rows[:, 0], tag=tag)
    pos = {}
    for g in np.unique(rows[:, 0]):
        pm = orc.perm(int(c["orders"][g]), F, H, W)
        inv = np.empty(N, np.int64)
        inv[pm] = np.arange(N)
        pos[g] = inv
    lg = np.array([lse_h[g, pos[g][n]] for g, n in rows])
    fin = np.isfinite(Lw)
    assert np.array_equal(fin, np.isfinite(lg))
    tol = LSE_ABS_F32_INPUT if cfg["dtype"] == "f32" else LSE_ABS
    lerr = np.max(np.abs(lg[fin] - Lw[fin])) if fin.any() else 0.0
    _say(f"  lse max_abs={lerr:.3e} (tol {tol})")
    assert lerr <= tol
    return On


def test_forward_tiny_static(bsa_gpu, orc):
    c = case(1)
    cfg = c["cfg"]
    rp, ci = _static_csr(cfg, c["seed"])
    rows = np.array([(g, n) for g in range(cfg["G"]) for n in range(cfg["N"])], np.int64)
    _say("[forward cfg 1 static 50%] all rows")
    _run_forward_case(bsa_gpu, orc, c, rp, ci, rows, tag="cfg1")


@pytest.mark.parametrize("dense", [False, True])
def test_forward_2k(bsa_gpu, orc, dense):
    c = case(2)
    cfg = c["cfg"]
    rp, ci = _static_csr(cfg, c["seed"], dense)
    rows = np.array([(g, n) for g in range(cfg["G"]) for n in range(0, cfg["N"], 3)], np.int64)
    _say(f"[forward cfg 2 {'100%' if dense else 'static 31%'}] {len(rows)} rows")
    _run_forward_case(bsa_gpu, orc, c, rp, ci, rows, tag=f"cfg2 dense={dense}")


@pytest.mark.parametrize("cid,rho", [(3, None), (4, None), (4, (20, 100)), (5, None)])
def test_forward_built_mask_full_size(bsa_gpu, orc, cid, rho):
    """Full-size configurations: the GPU runs its own mask end to end; the
    oracle builds its own mask and computes sampled rows."""
    c = case(cid)
    cfg = c["cfg"]
    F, H, W = cfg["F"], cfg["H"], cfg["W"]
    p = mask_params(bsa_gpu, cfg, rho)
    Qp, Kp, _ = gpu_reorder(bsa_gpu, c)
    grp, gci, gnnz = bsa_gpu.build_mask(Qp, Kp, c["orders_dev"], F, H, W, p)
    torch.cuda.synchronize()
    oq, ok_ = oracle_reorder(orc, c, "Q"), oracle_reorder(orc, c, "K")
    rp, ci = orc.build_mask(oq, ok_, F, H, W, c["orders"], p.Bq, p.Bk, p.score, p.rho_num,
                            p.rho_den, p.force_diag, p.win_T, p.win_r0)
    assert int(_np(gnnz)[0]) == len(ci)
    rows = sample_rows(cfg, c["orders"], orc, 192, c["seed"] + 7)
    _say(f"[forward cfg {cid} rho={rho}] density={len(ci) / (len(rp) - 1) / -(-cfg['N'] // p.Bk):.3f} "
         f"{len(rows)} sampled rows")
    _run_forward_case(bsa_gpu, orc, c, rp, ci, rows, gpu_mask=(grp, gci), tag=f"cfg{cid}")


# ------------------------------------------------------------ INT8 forward
def _int8_parity(bsa, orc, c, rp, ci, blocks, tag):
    cfg = c["cfg"]
    Bq, Bk, N = cfg["Bq"], cfg["Bk"], cfg["N"]
    Qp, Kp, Vp = gpu_reorder(bsa, c)
    (Qq, sQ), (Kq, sK), (Vq, sV) = (bsa.quantize_int8(x, B) for x, B in
                                    ((Qp, Bq), (Kp, Bk), (Vp, Bk)))
    grp, gci = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    Op, lse = bsa.forward_int8(Qq, sQ, Kq, sK, Vq, sV, grp, gci, Bq, Bk)
    torch.cuda.synchronize()
    oq = [orc.quantize_int8(oracle_reorder(orc, c, n), B)
          for n, B in (("Q", Bq), ("K", Bk), ("V", Bk))]
    Ow, Lw = orc.attention_int8(oq[0][0], oq[0][1], oq[1][0], oq[1][1], oq[2][0], oq[2][1], Bq, Bk,
                                rp, ci, blocks)
    Oh = _f64_from_bits(_bits(Op))
    Lh = _np(lse)
    got, want, heads, lg, lw = [], [], [], [], []
    for t, (g, i) in enumerate(blocks):
        nr = min(Bq, N - i * Bq)
        got.append(Oh[g, i * Bq:i * Bq + nr])
        want.append(Ow[t, :nr])
        heads += [g] * nr
        lg.append(Lh[g, i * Bq:i * Bq + nr])
        lw.append(Lw[t, :nr])
    _compare(np.concatenate(got), np.concatenate(want), heads=np.array(heads), tag=tag)
    lg, lw = np.concatenate(lg), np.concatenate(lw)
    assert np.max(np.abs(lg - lw)) <= LSE_ABS
    return Op


def test_forward_int8_2k(bsa_gpu, orc):
    c = case(2)
    cfg = c["cfg"]
    rp, ci = _static_csr(cfg, c["seed"])
    nq = -(-cfg["N"] // cfg["Bq"])
    blocks = np.array([(g, i) for g in range(cfg["G"]) for i in range(nq)], np.int64)
    _say("[int8 cfg 2] all blocks")
    _int8_parity(bsa_gpu, orc, c, rp, ci, blocks, "int8 cfg2")


@pytest.mark.parametrize("cid,rho,nb", [(3, None, 8), (4, None, 16), (4, (20, 100), 16)])
def test_forward_int8_full_size(bsa_gpu, orc, cid, rho, nb):
    c = case(cid)
    cfg = c["cfg"]
    F, H, W = cfg["F"], cfg["H"], cfg["W"]
    p = mask_params(bsa_gpu, cfg, rho)
    rp, ci = orc.build_mask(oracle_reorder(orc, c, "Q"), oracle_reorder(orc, c, "K"), F, H, W,
                            c["orders"], p.Bq, p.Bk, p.score, p.rho_num, p.rho_den, p.force_diag,
                            p.win_T, p.win_r0)
    nq = -(-cfg["N"] // cfg["Bq"])
    r = np.random.Generator(np.random.PCG64(c["seed"] + 11))
    blocks = [(int(r.integers(cfg["G"])), int(r.integers(nq))) for _ in range(nb - 3)]
    # first and ragged last q-block of the first and last head
    blocks += [(0, 0), (0, nq - 1), (cfg["G"] - 1, nq - 1)]
    blocks = np.array(blocks, np.int64)
    _say(f"[int8 cfg {cid} rho={p.rho_num}/{p.rho_den}] {len(blocks)} sampled q-blocks")
    _int8_parity(bsa_gpu, orc, c, rp, ci, blocks, f"int8 cfg{cid} rho={p.rho_num}")


@pytest.mark.parametrize("d,Bq,Bk", [(128, 128, 64), (128, 128, 128), (64, 64, 64), (64, 128, 64),
                                     (128, 64, 128)])
def test_int8_tiles_bit_exact(bsa_gpu, orc, d, Bq, Bk):
    """The INT8 kernel's own tile routines give the exact integer products."""
    G, N = 2, 300  # ragged: 300 = 2*128 + 44
    r = np.random.Generator(np.random.PCG64(d + Bq + Bk))
    Qq = r.integers(-127, 128, (G, N, d)).astype(np.int8)
    Kq = r.integers(-127, 128, (G, N, d)).astype(np.int8)
    Vq = r.integers(-127, 128, (G, N, d)).astype(np.int8)
    nq, nk = -(-N // Bq), -(-N // Bk)
    gij = np.array([(g, i, j) for g in range(G) for i in range(nq) for j in range(nk)], np.int32)
    S = bsa_gpu.debug_int8_qk(torch.from_numpy(Qq).cuda(), torch.from_numpy(Kq).cuda(),
                              torch.from_numpy(gij).cuda(), Bq, Bk)
    P8 = r.integers(0, 128, (len(gij), Bq, Bk)).astype(np.int8)
    gj = np.ascontiguousarray(gij[:, [0, 2]])
    OV = bsa_gpu.debug_int8_pv(torch.from_numpy(P8).cuda(), torch.from_numpy(Vq).cuda(),
                               torch.from_numpy(gj).cuda(), Bq, Bk)
    torch.cuda.synchronize()
    S, OV = _np(S), _np(OV)
    for t, (g, i, j) in enumerate(gij):
        assert np.array_equal(S[t], orc.int8_qk_tile(Qq, Kq, g, i, j, Bq, Bk)), (g, i, j)
        assert np.array_equal(OV[t], orc.int8_pv_tile(P8[t], Vq, g, j, Bq, Bk)), (g, j)


# ---------------------------------------------------- reference edge cases
def _forward_reordered_case(bsa, orc, Qn, Kn, Vn, rp, ci, F, H, W, Bq, Bk, tag):
    """Identity axis order: natural bf16 Q/K/V [N][G][d] -> reorder -> bf16
    forward with the given CSR -> inverse; every row against the oracle."""
    N, G, d = Qn.shape
    orders = np.zeros(G, np.uint8)
    od = torch.from_numpy(orders).cuda()
    dev = [torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda() for x in (Qn, Kn, Vn)]
    Qp, Kp, Vp = (bsa.permute(x, od, F, H, W, 0) for x in dev)
    Op, lse = bsa.forward(Qp, Kp, Vp, torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), Bq, Bk)
    O = bsa.permute(Op, od, F, H, W, 1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    host = [_bits(x) for x in dev]
    rows = np.array([(g, n) for g in range(G) for n in range(N)], np.int64)
    Ow, Lw = orc.attention_rows(*host, G, F, H, W, d, orders, rows, Bq, Bk, rp, ci)
    got = _np(O)[rows[:, 1], rows[:, 0]]
    _compare(got, Ow, heads=rows[:, 0], tag=tag)
    lg = _np(lse)[rows[:, 0], rows[:, 1]]
    assert np.max(np.abs(lg - Lw)) <= LSE_ABS


def test_forward_late_scores_far_above_reference(bsa_gpu, orc):
    """Keys of the last kv-block aligned with the queries of the second
    q-block: their scores exceed the reference taken from the first
    half-tile by ~140 (log2 units), so the kernel must take its exact path
    (row maxima first) for that workgroup.  Softmax then puts nearly all
    weight on the aligned keys, which the oracle also computes in fp64."""
    r = np.random.Generator(np.random.PCG64(31))
    F, H, W, G, d, Bq, Bk = 1, 4, 64, 2, 128, 128, 64
    N = F * H * W
    Q = r.standard_normal((N, G, d))
    K = r.standard_normal((N, G, d))
    V = r.standard_normal((N, G, d))
    u = r.standard_normal((G, d))
    Q[128:] = 3.0 * u[None] + 0.1 * r.standard_normal((N - 128, G, d))
    K[192:] = 3.0 * u[None] + 0.1 * r.standard_normal((N - 192, G, d))
    nq, nk = N // Bq, N // Bk
    rp = np.arange(0, G * nq * nk + 1, nk, dtype=np.int32)
    ci = np.tile(np.arange(nk, dtype=np.int32), G * nq)
    _forward_reordered_case(bsa_gpu, orc, Q, K, V, rp, ci, F, H, W, Bq, Bk, "late large scores")


def test_forward_first_half_tile_masked(bsa_gpu, orc):
    """N = 80 with 64-token blocks: the second q-block keeps only the ragged
    last kv-block (16 real keys), whose staged window starts at row 16, so
    the first 32-row half of that window is entirely masked and the row
    reference is only set by the second half."""
    r = np.random.Generator(np.random.PCG64(32))
    F, H, W, G, d, Bq, Bk = 1, 1, 80, 1, 64, 64, 64
    N = F * H * W
    Q, K, V = (r.standard_normal((N, G, d)) for _ in range(3))
    rp = np.array([0, 2, 3], np.int32)
    ci = np.array([0, 1, 1], np.int32)
    _forward_reordered_case(bsa_gpu, orc, Q, K, V, rp, ci, F, H, W, Bq, Bk, "masked first half")


# ------------------------------------------------------------ edge cases
@pytest.mark.parametrize("N,d", [(40, 64), (40, 128), (1, 128), (63, 64)])
def test_forward_fewer_tokens_than_a_sub_tile(bsa_gpu, orc, N, d):
    """N below the 64-row staging window (the clamped-row variant of the
    kernel): one q-block, one kv-block, every row against the oracle."""
    r = np.random.Generator(np.random.PCG64(40 + N + d))
    G = 2
    Q, K, V = (r.standard_normal((N, G, d)) for _ in range(3))
    rp = np.array([0, 1, 2], np.int32)
    ci = np.array([0, 0], np.int32)
    _forward_reordered_case(bsa_gpu, orc, Q, K, V, rp, ci, 1, 1, N, 64, 64, f"N={N} d={d}")


def test_forward_empty_rows_and_out_of_range_entries(bsa_gpu, orc):
    """Rows with no kept block give O = 0 and lse = -inf; CSR entries outside
    [0, Nkv) are skipped."""
    r = np.random.Generator(np.random.PCG64(41))
    F, H, W, G, d, B = 1, 4, 64, 2, 128, 64
    N = F * H * W
    Q, K, V = (r.standard_normal((N, G, d)) for _ in range(3))
    nq = N // B
    # head 0: rows 0 and 2 empty; head 1: row 1 keeps an out-of-range entry only
    rows_sets = [[], [0, 1], [], [3], [0, 2], [99], [1, 3], [-5, 2]]
    rp = np.cumsum([0] + [len(s) for s in rows_sets]).astype(np.int32)
    ci = np.array([j for s in rows_sets for j in s], np.int32)
    od = torch.zeros(G, dtype=torch.uint8).cuda()
    dev = [torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda() for x in (Q, K, V)]
    Qp, Kp, Vp = (bsa_gpu.permute(x, od, F, H, W, 0) for x in dev)
    Op, lse = bsa_gpu.forward(Qp, Kp, Vp, torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(),
                              B, B)
    torch.cuda.synchronize()
    o, l = _np(Op.float()), _np(lse)
    host = [_bits(x) for x in dev]
    rows = np.array([(g, n) for g in range(G) for n in range(N)], np.int64)
    Ow, Lw = orc.attention_rows(*host, G, F, H, W, d, np.zeros(G, np.uint8), rows, B, B, rp, ci)
    got = o[rows[:, 0], rows[:, 1]]
    empty = ~np.isfinite(Lw)
    assert empty.sum() == 3 * B  # rows 0 and 2 of head 0, row 1 of head 1
    assert np.all(got[empty] == 0.0) and np.all(np.isneginf(l[rows[empty, 0], rows[empty, 1]]))
    _compare(got[~empty], Ow[~empty], tag="non-empty rows")


def test_forward_mask_shared_across_heads(bsa_gpu, orc):
    """mask_G < G: head g reads CSR rows (g % mask_G) * Nq + i (batch copies
    sharing one mask), for the bf16 and the INT8 forward."""
    r = np.random.Generator(np.random.PCG64(42))
    F, H, W, G, d, B, mG = 1, 8, 64, 4, 64, 64, 2
    N = F * H * W
    nq = N // B
    Q, K, V = (r.standard_normal((N, G, d)) for _ in range(3))
    sets = [sorted(set(r.choice(nq, size=3, replace=False).tolist()) | {i % nq})
            for i in range(mG * nq)]
    rp = np.cumsum([0] + [len(s) for s in sets]).astype(np.int32)
    ci = np.array([j for s in sets for j in s], np.int32)
    od = torch.zeros(G, dtype=torch.uint8).cuda()
    dev = [torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda() for x in (Q, K, V)]
    Qp, Kp, Vp = (bsa_gpu.permute(x, od, F, H, W, 0) for x in dev)
    grp, gci = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    Op, lse = bsa_gpu.forward(Qp, Kp, Vp, grp, gci, B, B, mask_G=mG)
    torch.cuda.synchronize()
    host = [_bits(x) for x in dev]
    rows = np.array([(g, n) for g in range(G) for n in range(N)], np.int64)
    Ow, Lw = orc.attention_rows(*host, G, F, H, W, d, np.zeros(G, np.uint8), rows, B, B, rp, ci,
                                mask_G=mG)
    _compare(_np(Op.float())[rows[:, 0], rows[:, 1]], Ow, heads=rows[:, 0], tag="shared mask")
    # INT8: the same sharing against the INT8 emulation (the oracle quantises
    # the same bf16 inputs with its own quantiser)
    (qq, sq), (kq, sk), (vq, sv) = (bsa_gpu.quantize_int8(x, B) for x in (Qp, Kp, Vp))
    O8, _ = bsa_gpu.forward_int8(qq, sq, kq, sk, vq, sv, grp, gci, B, B, mask_G=mG)
    torch.cuda.synchronize()
    blocks = np.array([(g, i) for g in range(G) for i in range(nq)], np.int64)
    # identity order: the reordered tensors are the natural ones, head-major
    oq = [orc.quantize_int8(np.ascontiguousarray(h.reshape(N, G, d).transpose(1, 0, 2)), B)
          for h in host]
    W8, _ = orc.attention_int8(oq[0][0], oq[0][1], oq[1][0], oq[1][1], oq[2][0], oq[2][1], B, B,
                               rp, ci, blocks, mask_G=mG)
    o8 = _np(O8.float())
    got8 = np.concatenate([o8[g, i * B:(i + 1) * B] for g, i in blocks])
    _compare(got8, W8.reshape(-1, d), tag="shared mask int8")


@pytest.mark.parametrize("N,d,Bq,Bk", [(40, 64, 64, 64), (1, 128, 128, 64), (100, 128, 128, 128)])
def test_forward_int8_short_sequences(bsa_gpu, orc, N, d, Bq, Bk):
    """INT8 forward when the sequence is shorter than a tile (rows and
    columns past N read as zero and are masked) against the INT8 emulation."""
    r = np.random.Generator(np.random.PCG64(43 + N))
    G = 2
    x = [torch.from_numpy(r.standard_normal((G, N, d)).astype(np.float32)).to(torch.bfloat16).cuda()
         for _ in range(3)]
    (qq, sq), (kq, sk), (vq, sv) = (bsa_gpu.quantize_int8(t, B) for t, B in zip(x, (Bq, Bk, Bk)))
    nq, nk = -(-N // Bq), -(-N // Bk)
    rp = np.arange(0, G * nq * nk + 1, nk, dtype=np.int32)
    ci = np.tile(np.arange(nk, dtype=np.int32), G * nq)
    O8, _ = bsa_gpu.forward_int8(qq, sq, kq, sk, vq, sv, torch.from_numpy(rp).cuda(),
                                 torch.from_numpy(ci).cuda(), Bq, Bk)
    torch.cuda.synchronize()
    blocks = np.array([(g, i) for g in range(G) for i in range(nq)], np.int64)
    # the oracle quantises the same bf16 inputs with its own quantiser
    oq = [orc.quantize_int8(_bits(t), B) for t, B in zip(x, (Bq, Bk, Bk))]
    W8, _ = orc.attention_int8(oq[0][0], oq[0][1], oq[1][0], oq[1][1], oq[2][0], oq[2][1], Bq, Bk,
                               rp, ci, blocks)
    o8 = _np(O8.float())
    got = np.concatenate([o8[g, i * Bq:min((i + 1) * Bq, N)] for g, i in blocks])
    want = np.concatenate([W8[t, :min(Bq, N - i * Bq)] for t, (g, i) in enumerate(blocks)])
    _compare(got, want, tag=f"int8 N={N}")
