"""GPU coverage beyond the per-configuration parity runs:

* every (d, Bq, Bk) forward instantiation the C ABI accepts, bf16 and INT8,
  on a short sequence with a ragged tail, against the oracle;
* INT8 with large score scales (wide Q / K ranges and single outliers), where
  the tile maximum's code must stay at 127, and at the largest integer tile
  products (every code at its bound);
* run-to-run bitwise equality of both forwards at the 480p shape;
* guard regions around every output buffer (O natural and reordered, lse,
  row_ptr, col_idx, nnz, INT8 codes and scales, block sums), which must be
  unchanged after the calls.

The oracle quantises its own inputs (from the same bf16 values); nothing it
compares against comes from the HIP path.
"""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_ABS = 2e-2
LSE_ABS = 1e-3
LSE_REL = 2.0 ** -21


def _say(msg):
    print(msg, flush=True)


def _np(t):
    return t.detach().cpu().numpy()


def _bits(t):
    from block_sparse_attention_inverse_amd import synth

    return synth.bf16_bits(t)


def _compare(got, want, tag, heads=None):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    diff = got - want
    rel = np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-30)
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    _say(f"  {tag}: rel_l2={rel:.3e} max_abs={mx:.3e} n={diff.shape[0]}")
    assert np.all(np.isfinite(got)), tag
    assert rel <= REL_L2, f"{tag}: rel L2 {rel}"
    assert mx <= MAX_ABS, f"{tag}: max abs {mx}"
    if heads is not None:
        for g in np.unique(heads):
            sel = heads == g
            rg = np.linalg.norm(diff[sel]) / max(np.linalg.norm(want[sel]), 1e-30)
            assert rg <= REL_L2, f"{tag}: head {g} rel L2 {rg}"


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).cuda()


def _int8_all_blocks(bsa, orc, Qp, Kp, Vp, rp, ci, Bq, Bk, tag, host_p):
    """GPU: quantise reordered bf16 Qp/Kp/Vp [G][N][d] and run the INT8
    forward; oracle: its own quantiser on host_p, the same bf16 values in the
    same [G][N][d] order held on the host (the inputs themselves, or the
    oracle's own reorder of them), then the INT8 emulation on every q-block.
    Returns the GPU output."""
    G, N, d = Qp.shape
    (qq, sq), (kq, sk), (vq, sv) = (bsa.quantize_int8(x, B) for x, B in ((Qp, Bq), (Kp, Bk), (Vp, Bk)))
    O8, L8 = bsa.forward_int8(qq, sq, kq, sk, vq, sv, torch.from_numpy(rp).cuda(),
                              torch.from_numpy(ci).cuda(), Bq, Bk)
    torch.cuda.synchronize()
    oq = [orc.quantize_int8(x, B) for x, B in zip(host_p, (Bq, Bk, Bk))]
    nq = -(-N // Bq)
    blocks = np.array([(g, i) for g in range(G) for i in range(nq)], np.int64)
    Ow, Lw = orc.attention_int8(oq[0][0], oq[0][1], oq[1][0], oq[1][1], oq[2][0], oq[2][1], Bq, Bk,
                                rp, ci, blocks)
    o8, l8 = _np(O8.float()), _np(L8)
    got = np.concatenate([o8[g, i * Bq:min((i + 1) * Bq, N)] for g, i in blocks])
    want = np.concatenate([Ow[t, :min(Bq, N - i * Bq)] for t, (g, i) in enumerate(blocks)])
    heads = np.concatenate([[g] * min(Bq, N - i * Bq) for g, i in blocks])
    _compare(got, want, tag, heads=heads)
    lg = np.concatenate([l8[g, i * Bq:min((i + 1) * Bq, N)] for g, i in blocks])
    lw = np.concatenate([Lw[t, :min(Bq, N - i * Bq)] for t, (g, i) in enumerate(blocks)])
    fin = np.isfinite(lw)
    assert np.array_equal(fin, np.isfinite(lg))
    # the kernel's lse is an fp32 value: beside the absolute 1e-3 it carries
    # a few fp32 ulps of its own magnitude (the large-scale cases reach 4e4)
    tol = LSE_ABS + LSE_REL * np.abs(lw[fin])
    assert np.all(np.abs(lg[fin] - lw[fin]) <= tol)
    return O8


# ------------------------------------------------- every forward instantiation
INSTANTIATIONS = [(d, bq, bk) for d in (64, 128) for bq in (64, 128) for bk in (64, 128)]


@pytest.mark.parametrize("d,Bq,Bk", INSTANTIATIONS)
def test_forward_every_instantiation(bsa_gpu, orc, d, Bq, Bk):
    """bf16 and INT8 forwards of one (d, Bq, Bk) kernel on a 2 x 4 x 53 grid
    (N = 424: ragged last q- and kv-block for every block size), two heads
    with different axis orders, a static mask with the diagonal and about half
    of the kv-blocks; every row against the oracle."""
    from block_sparse_attention_inverse_amd import synth

    F, H, W, G = 2, 4, 53, 2
    N = F * H * W
    r = np.random.Generator(np.random.PCG64(600 + d + Bq + 3 * Bk))
    orders = np.array([1, 4], np.uint8)
    od = torch.from_numpy(orders).cuda()
    nat = [r.standard_normal((N, G, d)).astype(np.float32) for _ in range(3)]
    nq, nk = -(-N // Bq), -(-N // Bk)
    rp, ci = synth.static_mask(G, N, Bq, Bk, max(1, nk // 2), 700 + d + Bq + Bk)
    dev = [_bf16(x) for x in nat]
    Qp, Kp, Vp = (bsa_gpu.permute(x, od, F, H, W, 0) for x in dev)
    _say(f"[instantiation d={d} Bq={Bq} Bk={Bk}] N={N} nq={nq} nk={nk} nnz={len(ci)}")
    # bf16, output written in natural order by the epilogue
    O, lse = bsa_gpu.forward_natural(Qp, Kp, Vp, torch.from_numpy(rp).cuda(),
                                     torch.from_numpy(ci).cuda(), Bq, Bk, od, F, H, W)
    torch.cuda.synchronize()
    host = [_bits(x) for x in dev]
    rows = np.array([(g, n) for g in range(G) for n in range(N)], np.int64)
    Ow, Lw = orc.attention_rows(*host, G, F, H, W, d, orders, rows, Bq, Bk, rp, ci)
    _compare(_np(O.float())[rows[:, 1], rows[:, 0]], Ow, f"bf16 d={d} {Bq}x{Bk}", heads=rows[:, 0])
    lg = _np(lse)[rows[:, 0], rows[:, 1]]
    assert np.max(np.abs(lg - Lw)) <= LSE_ABS
    # INT8 on the reordered tensors (the oracle reorders the host bits itself)
    host_p = [orc.permute(0, h, np.uint16, G, F, H, W, d, orders) for h in host]
    _int8_all_blocks(bsa_gpu, orc, Qp, Kp, Vp, rp, ci, Bq, Bk, f"int8 d={d} {Bq}x{Bk}", host_p)


# ------------------------------------------------- INT8 with large score scales
@pytest.mark.parametrize("kind,scale", [("uniform", 40.0), ("uniform", 100.0), ("outlier", 60.0),
                                        ("outlier", 120.0)])
def test_int8_large_score_scales(bsa_gpu, orc, kind, scale):
    """Score scales f = sQ sK sm_scale log2(e) far above those of unit-normal
    inputs.  'uniform': Q and K scaled as a whole (softmax nearly one-hot);
    'outlier': unit-normal Q and K with one large channel value per block, so
    the per-block scale is large while the softmax stays spread.  The tile
    maximum's code must come out as 127 (a code of 128 reads as -128 in the
    signed product and flips the output's sign)."""
    G, N, d, Bq, Bk = 2, 300, 128, 128, 64
    r = np.random.Generator(np.random.PCG64(800 + int(scale)))
    Q, K, V = (r.standard_normal((G, N, d)).astype(np.float32) for _ in range(3))
    if kind == "uniform":
        Q *= scale
        K *= scale
    else:
        for X, B in ((Q, Bq), (K, Bk)):
            for b0 in range(0, N, B):
                X[:, b0 + int(r.integers(min(B, N - b0))), int(r.integers(d))] = scale
    Qp, Kp, Vp = (_bf16(x) for x in (Q, K, V))
    host_p = [orc.f32_to_bf16(x) for x in (Q, K, V)]
    nq, nk = -(-N // Bq), -(-N // Bk)
    rp = np.arange(0, G * nq * nk + 1, nk, dtype=np.int32)
    ci = np.tile(np.arange(nk, dtype=np.int32), G * nq)
    _say(f"[int8 large scales {kind} x{scale}]")
    _int8_all_blocks(bsa_gpu, orc, Qp, Kp, Vp, rp, ci, Bq, Bk, f"int8 {kind} x{scale}", host_p)


# ------------------------------------------------- INT8 at the product bound
@pytest.mark.parametrize("Bk", [64, 128])
def test_int8_extreme_tile_products(bsa_gpu, orc, Bk):
    """Every code at its largest magnitude: Q = 0 makes every score 0, so
    every P8 code is 127, and V is +0.5 in one head and -0.5 in the other, so
    every V8 code is +-127.  Each full tile's integer product then reaches
    +-Bk * 127 * 127, the bound the kernel's biased fp32 read of the product
    tiles relies on, and every output element must be +-0.5 (the last,
    ragged kv-block has fewer real columns)."""
    G, N, d, Bq = 2, 500, 128, 128
    r = np.random.Generator(np.random.PCG64(900 + Bk))
    Q = np.zeros((G, N, d), np.float32)
    K = r.standard_normal((G, N, d)).astype(np.float32)
    V = np.empty((G, N, d), np.float32)
    V[0], V[1] = 0.5, -0.5
    Qp, Kp, Vp = (_bf16(x) for x in (Q, K, V))
    host_p = [orc.f32_to_bf16(x) for x in (Q, K, V)]
    nq, nk = -(-N // Bq), -(-N // Bk)
    rp = np.arange(0, G * nq * nk + 1, nk, dtype=np.int32)
    ci = np.tile(np.arange(nk, dtype=np.int32), G * nq)
    _say(f"[int8 extreme products Bk={Bk}]")
    O8 = _int8_all_blocks(bsa_gpu, orc, Qp, Kp, Vp, rp, ci, Bq, Bk, f"int8 extreme Bk={Bk}", host_p)
    o8 = _np(O8.float())
    assert np.array_equal(o8[0], np.full((N, d), 0.5, np.float32))
    assert np.array_equal(o8[1], np.full((N, d), -0.5, np.float32))


# ------------------------------------------------- determinism
def test_forwards_bitwise_deterministic(bsa_gpu):
    """Two runs of the bf16 and of the INT8 forward (natural-order output) on
    the 480p layer with its built mask give identical bits (O and lse)."""
    from block_sparse_attention_inverse_amd import synth

    cfg = synth.config(3)
    seed = synth.seed_of(3)
    F, H, W = cfg["F"], cfg["H"], cfg["W"]
    orders = synth.make_orders(cfg, seed)
    od = torch.from_numpy(orders).cuda()
    Q, K, V = synth.cast_inputs(cfg, *synth.make_qkv(cfg, orders, seed, device="cuda"))
    p = bsa_gpu.mask_params(cfg["Bq"], cfg["Bk"], 0, cfg["rho"], True)
    Qp, Kp, Vp = (bsa_gpu.permute(x, od, F, H, W, 0) for x in (Q, K, V))
    rp, ci, nnz = bsa_gpu.build_mask(Qp, Kp, od, F, H, W, p)
    rp2, ci2, nnz2 = bsa_gpu.build_mask(Qp, Kp, od, F, H, W, p)
    n = int(nnz.item())
    assert n == int(nnz2.item())
    assert torch.equal(rp, rp2) and torch.equal(ci[:n], ci2[:n])  # entries past nnz are unused
    _say("[determinism 480p] bf16")
    outs = [bsa_gpu.forward_natural(Qp, Kp, Vp, rp, ci, p.Bq, p.Bk, od, F, H, W) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    _say("[determinism 480p] int8")
    q8 = [bsa_gpu.quantize_int8(x, B) for x, B in ((Qp, p.Bq), (Kp, p.Bk), (Vp, p.Bk))]
    args = [t for pair in q8 for t in pair]
    o8 = [bsa_gpu.forward_int8_natural(*args, rp, ci, p.Bq, p.Bk, od, F, H, W) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(o8[0][0], o8[1][0]) and torch.equal(o8[0][1], o8[1][1])


# ------------------------------------------------- guard regions
GUARD_BYTES = 4096


class Guarded:
    """A device buffer of ``n`` elements with GUARD_BYTES of a fixed pattern
    before and after it; ``view`` is the payload."""

    def __init__(self, n, dtype, shape=None):
        es = torch.empty((), dtype=dtype).element_size()
        self.g = GUARD_BYTES // es
        self.buf = torch.empty(n + 2 * self.g, dtype=dtype, device="cuda")
        raw = self.buf.view(torch.uint8)
        pat = torch.tensor([0xA5, 0x3C, 0x5A, 0xC3], dtype=torch.uint8, device="cuda")
        raw.copy_(pat.repeat(-(-raw.numel() // 4))[:raw.numel()])
        self.before = raw.clone()
        self.view = self.buf[self.g:self.g + n]
        if shape is not None:
            self.view = self.view.view(*shape)
        self.nbytes = n * es

    def check(self, tag):
        raw = self.buf.view(torch.uint8)
        ge = GUARD_BYTES
        assert torch.equal(raw[:ge], self.before[:ge]), f"{tag}: guard before the buffer changed"
        assert torch.equal(raw[ge + self.nbytes:], self.before[ge + self.nbytes:]), \
            f"{tag}: guard after the buffer changed"


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_outputs_stay_inside_their_buffers(bsa_gpu):
    """Every entry point of the chain writes only inside its output buffers:
    fused reorder (bf16 copy, block sums, INT8 codes and scales), mask build
    (row_ptr, col_idx, nnz), bf16 and INT8 forwards in reordered and natural
    order (O, lse), inverse reorder; ragged 2k-shaped layer plus a 480p one."""
    from block_sparse_attention_inverse_amd import _lib, synth

    lib = _lib.load()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for cid in (2, 3):
        cfg = synth.config(cid)
        seed = synth.seed_of(cid)
        F, H, W, G, d, N = cfg["F"], cfg["H"], cfg["W"], cfg["G"], cfg["d"], cfg["N"]
        Bq, Bk = cfg["Bq"], cfg["Bk"]
        nq, nk = -(-N // Bq), -(-N // Bk)
        orders = synth.make_orders(cfg, seed)
        od = torch.from_numpy(orders).cuda()
        Q, K, V = synth.cast_inputs(cfg, *synth.make_qkv(cfg, orders, seed, device="cuda"))
        _say(f"[guards cfg {cid}] N={N} G={G} d={d}")
        bufs = {}
        outs = {}
        for name, X, B in (("Q", Q, Bq), ("K", K, Bk), ("V", V, Bk)):
            xp = Guarded(G * N * d, torch.bfloat16, (G, N, d))
            sums = Guarded(G * -(-N // B) * d, torch.float32)
            xq = Guarded(G * N * d, torch.int8)
            sc = Guarded(G * -(-N // B), torch.float32)
            rc = lib.bsa_permute_pool(_p(X), _lib.BSA_BF16, _p(xp.view), X.stride(1), X.stride(0), G,
                                      F, H, W, d, _p(od), B, _p(sums.view), _p(xq.view),
                                      _p(sc.view), st)
            _lib.check(rc)
            bufs.update({f"{name}p": xp, f"{name}sums": sums, f"{name}q": xq, f"{name}s": sc})
            outs[name] = (xp.view, sums.view, xq.view, sc.view)
        p = bsa_gpu.mask_params(Bq, Bk, 0, cfg.get("rho", (30, 100)), True)
        cap = bsa_gpu.mask_capacity(G, F, H, W, p)
        ws = torch.empty(bsa_gpu.mask_workspace(G, F, H, W, d, p), dtype=torch.uint8, device="cuda")
        rp = Guarded(G * nq + 1, torch.int32)
        ci = Guarded(cap, torch.int32)
        nnz = Guarded(1, torch.int32)
        _lib.check(lib.bsa_build_mask_pooled(_p(outs["Q"][1]), _p(outs["K"][1]), G, F, H, W, d,
                                             _p(od), ctypes.byref(p), _p(rp.view), _p(ci.view), cap,
                                             _p(nnz.view), _p(ws), ws.numel(), st))
        bufs.update(row_ptr=rp, col_idx=ci, nnz=nnz)
        Qp, Kp, Vp = outs["Q"][0], outs["K"][0], outs["V"][0]
        for nat in (False, True):
            for int8 in (False, True):
                o = Guarded(G * N * d, torch.bfloat16)
                lse = Guarded(G * N, torch.float32)
                if int8:
                    qa = [outs[n][2] for n in "QKV"]
                    sa = [outs[n][3] for n in "QKV"]
                    head = [_p(qa[0]), _p(sa[0]), _p(qa[1]), _p(sa[1]), _p(qa[2]), _p(sa[2])]
                else:
                    head = [_p(Qp), _p(Kp), _p(Vp)]
                if nat:
                    fn = lib.bsa_forward_int8_natural if int8 else lib.bsa_forward_natural
                    rc = fn(*head, _p(rp.view), _p(ci.view), cap, G, _p(od), F, H, W, _p(o.view), d,
                            G * d, _p(lse.view), G, d, Bq, Bk, ctypes.c_float(0.0), st)
                else:
                    fn = lib.bsa_forward_int8 if int8 else lib.bsa_forward
                    rc = fn(*head, _p(rp.view), _p(ci.view), cap, G, _p(o.view), _p(lse.view), G, N,
                            d, Bq, Bk, ctypes.c_float(0.0), st)
                _lib.check(rc)
                bufs[f"O nat={nat} int8={int8}"] = o
                bufs[f"lse nat={nat} int8={int8}"] = lse
        back = Guarded(N * G * d, torch.bfloat16)
        _lib.check(lib.bsa_permute(1, _p(Qp), _lib.BSA_BF16, _p(back.view), _lib.BSA_BF16, d, G * d,
                                   G, F, H, W, d, _p(od), st))
        bufs["inverse reorder"] = back
        torch.cuda.synchronize()
        assert torch.equal(back.view.view(N, G, d), Q)
        for tag, b in bufs.items():
            b.check(f"cfg {cid} {tag}")
