"""Seeded synthetic workloads with the shapes of the pages' video DiT layers.

This module generates inputs only (Q/K/V, per-head axis orders, static
block masks); it holds none of the method's arithmetic and is shared by the
tests, the benchmark and the smoke check.  The pages measure on real models
and prompt suites that are not available here; these tensors stand in for
them with the same token grids, head counts, head dim and density range.

Recipe (per configuration, seed = 1000 + config id unless given):
  * orders: one of the six F/H/W axis orders per head, uniform (numpy
    PCG64); the long-clip configuration uses frame-major order for every
    head (its temporal window is defined on frames).
  * Q, K, V natural order [N][G][d]: iid N(0,1) plus a shared smooth local
    component L_g: N(0,1) noise on the [F][H][W][d] grid, box-averaged with
    half-width 3 along the head's innermost axis, 1 along the middle axis,
    0 along the outermost (clamped at the edges), normalised to unit std and
    scaled by 0.5.  Q = Xq + L, K = Xk + L, V = Xv + 0.5 L.  This gives
    peaked, local attention after reordering, and keeps |V| well below 8.
  * dtype: the tiny configuration stays fp32; the others are rounded to
    bf16 (round-to-nearest-even, torch's conversion).
  * static masks (tiny and 2k configurations): per row, the diagonal block
    plus k-1 other blocks drawn without replacement, ascending.
"""
import numpy as np
import torch

CONFIGS = {
    1: dict(name="tiny", F=4, H=8, W=8, G=2, d=64, dtype="f32", Bq=64, Bk=64, mask="static",
            k_static=2),
    2: dict(name="2k", F=8, H=16, W=16, G=8, d=64, dtype="bf16", Bq=64, Bk=64, mask="static",
            k_static=10),
    3: dict(name="480p", F=21, H=30, W=52, G=12, d=128, dtype="bf16", Bq=128, Bk=64, mask="dot",
            rho=(30, 100)),
    4: dict(name="720p", F=21, H=45, W=80, G=40, d=128, dtype="bf16", Bq=128, Bk=64, mask="dot",
            rho=(30, 100)),
    5: dict(name="long", F=33, H=45, W=80, G=24, d=128, dtype="bf16", Bq=128, Bk=128,
            mask="cosine", rho=(15, 100), win_T=2, win_r0=4, frame_major=True),
}

# axis-order code -> (outermost, middle, innermost) axis, axes 0=F, 1=H, 2=W
_ORDER_AXES = {0: (0, 1, 2), 1: (0, 2, 1), 2: (1, 0, 2), 3: (1, 2, 0), 4: (2, 0, 1), 5: (2, 1, 0)}


def config(cid: int, **over) -> dict:
    c = dict(CONFIGS[cid])
    c["id"] = cid
    c.update(over)
    c["N"] = c["F"] * c["H"] * c["W"]
    return c


def seed_of(cid: int) -> int:
    return 1000 + cid


def make_orders(cfg: dict, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    if cfg.get("frame_major"):
        return np.zeros(cfg["G"], dtype=np.uint8)
    return rng.integers(0, 6, size=cfg["G"]).astype(np.uint8)


def _box_mean(x: torch.Tensor, dim: int, hw: int) -> torch.Tensor:
    if hw == 0:
        return x
    n = x.shape[dim]
    c = torch.cumsum(x, dim)
    zshape = list(x.shape)
    zshape[dim] = 1
    c = torch.cat([torch.zeros(zshape, dtype=x.dtype, device=x.device), c], dim)
    idx = torch.arange(n, device=x.device)
    hi = torch.clamp(idx + hw, max=n - 1) + 1
    lo = torch.clamp(idx - hw, min=0)
    s = c.index_select(dim, hi) - c.index_select(dim, lo)
    shape = [1] * x.dim()
    shape[dim] = n
    return s / (hi - lo).to(x.dtype).reshape(shape)


def make_qkv(cfg: dict, orders: np.ndarray, seed: int, device="cpu", heads=None):
    """Natural-order fp32 Q, K, V [N][G][d] on ``device`` (torch RNG seeded
    by ``seed``).  ``heads`` restricts the local component to those heads
    (others still get it; the argument only exists for partial generation)."""
    F, H, W, G, d = cfg["F"], cfg["H"], cfg["W"], cfg["G"], cfg["d"]
    N = F * H * W
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    Q = torch.randn((N, G, d), generator=gen, device=device, dtype=torch.float32)
    K = torch.randn((N, G, d), generator=gen, device=device, dtype=torch.float32)
    V = torch.randn((N, G, d), generator=gen, device=device, dtype=torch.float32)
    for g in range(G):
        outer, mid, inner = _ORDER_AXES[int(orders[g])]
        z = torch.randn((F, H, W, d), generator=gen, device=device, dtype=torch.float32)
        z = _box_mean(z, inner, 3)
        z = _box_mean(z, mid, 1)
        z = z / z.std()
        L = (0.5 * z).reshape(N, d)
        Q[:, g, :] += L
        K[:, g, :] += L
        V[:, g, :] += 0.5 * L
    return Q, K, V


def cast_inputs(cfg: dict, Q, K, V):
    if cfg["dtype"] == "f32":
        return Q, K, V
    return Q.to(torch.bfloat16), K.to(torch.bfloat16), V.to(torch.bfloat16)


def diag_blocks(i: int, N: int, Bq: int, Bk: int):
    """kv-blocks whose token range overlaps q-block i's range."""
    q0, q1 = i * Bq, min((i + 1) * Bq, N)
    return list(range(q0 // Bk, (q1 - 1) // Bk + 1))


def static_mask(G: int, N: int, Bq: int, Bk: int, k: int, seed: int):
    """Random static CSR: per row the diagonal block(s) plus k - |diag| other
    blocks without replacement, ascending.  Returns numpy int32 (row_ptr, col_idx)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nq, nk = -(-N // Bq), -(-N // Bk)
    rows = []
    for _g in range(G):
        for i in range(nq):
            dg = diag_blocks(i, N, Bq, Bk)
            rest = np.setdiff1d(np.arange(nk), dg)
            extra = max(0, min(k - len(dg), rest.size))
            pick = rng.choice(rest, size=extra, replace=False) if extra else np.empty(0, np.int64)
            rows.append(np.sort(np.concatenate([np.asarray(dg, np.int64), pick])))
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum([r.size for r in rows])
    col_idx = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    return row_ptr, col_idx


def dense_mask(G: int, N: int, Bq: int, Bk: int):
    nq, nk = -(-N // Bq), -(-N // Bk)
    row_ptr = (np.arange(G * nq + 1, dtype=np.int64) * nk).astype(np.int32)
    col_idx = np.tile(np.arange(nk, dtype=np.int32), G * nq)
    return row_ptr, col_idx


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
