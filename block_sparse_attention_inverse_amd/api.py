"""Python binding of the C ABI in include/bsa.h, on torch device tensors.

Each function checks tensor properties, passes raw device pointers and the
current HIP stream to the C entry point of the same name, and allocates its
outputs with torch (torch is only the allocator and stream provider here).
Every step of the computation runs in the HIP kernels of libbsa.so.
"""
import ctypes

import torch

from . import _lib
from ._lib import MaskParams, BSA_BF16, BSA_F32, check

_DT = {torch.float32: BSA_F32, torch.bfloat16: BSA_BF16, torch.int8: _lib.BSA_I8}


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("bsa: tensors must live on the GPU")


def abi_version() -> int:
    return int(_lib.load().bsa_abi_version())


def last_error() -> str:
    m = _lib.load().bsa_last_error()
    return m.decode() if m else ""


def mask_params(Bq=64, Bk=64, score=0, rho=(30, 100), force_diag=True, win_T=-1, win_r0=0):
    return MaskParams(Bq, Bk, score, rho[0], rho[1], 1 if force_diag else 0, win_T, win_r0)


def permute(x, axis_order, F, H, W, direction=0, out=None, out_dtype=torch.bfloat16):
    """bsa_permute.  direction 0: natural x [N][G][d] (any strides with unit
    channel stride) -> reordered [G][N][d]; direction 1: reordered x [G][N][d]
    -> natural (``out`` may be a strided [N][G][d] view; default new [N][G][d]).
    ``axis_order``: uint8 device tensor [G]."""
    _lib.load()
    N = F * H * W
    if direction == 0:
        if x.dim() != 3 or x.shape[0] != N or x.stride(2) != 1:
            raise ValueError("natural input must be [N][G][d] with unit channel stride")
        G, d = x.shape[1], x.shape[2]
        sn, sg = x.stride(0), x.stride(1)
        if out is None:
            out = torch.empty((G, N, d), dtype=out_dtype, device=x.device)
        src, dst = x, out
    else:
        if x.dim() != 3 or x.shape[1] != N or not x.is_contiguous():
            raise ValueError("reordered input must be contiguous [G][N][d]")
        G, d = x.shape[0], x.shape[2]
        if out is None:
            out = torch.empty((N, G, d), dtype=out_dtype, device=x.device)
        if out.shape != (N, G, d) or out.stride(2) != 1:
            raise ValueError("natural output must be [N][G][d] with unit channel stride")
        sn, sg = out.stride(0), out.stride(1)
        src, dst = x, out
    _dev(src, dst, axis_order)
    if axis_order.dtype != torch.uint8 or axis_order.numel() < G:
        raise ValueError("axis_order must be a uint8 tensor with G entries")
    rc = _lib.load().bsa_permute(direction, _ptr(src), _DT[src.dtype], _ptr(dst), _DT[dst.dtype],
                                 sg, sn, G, F, H, W, d, _ptr(axis_order), _stream())
    check(rc)
    return out


def mask_capacity(G, F, H, W, params: MaskParams) -> int:
    v = int(_lib.load().bsa_mask_capacity(G, F, H, W, ctypes.byref(params)))
    if v < 0:
        check(v)
    return v


def mask_workspace(G, F, H, W, d, params: MaskParams) -> int:
    v = int(_lib.load().bsa_mask_workspace(G, F, H, W, d, ctypes.byref(params)))
    if v < 0:
        check(v)
    return v


def build_mask(Qp, Kp, axis_order, F, H, W, params: MaskParams, workspace=None):
    """bsa_build_mask on reordered bf16 Qp, Kp [G][N][d].  Returns
    (row_ptr int32[G*Nq+1], col_idx int32[capacity], nnz int32[1]) on the
    device; only col_idx[:nnz] is meaningful."""
    _dev(Qp, Kp, axis_order)
    G, N, d = Qp.shape
    cap = mask_capacity(G, F, H, W, params)
    ws_bytes = mask_workspace(G, F, H, W, d, params)
    nq = (N + params.Bq - 1) // params.Bq
    row_ptr = torch.empty(G * nq + 1, dtype=torch.int32, device=Qp.device)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=Qp.device)
    nnz = torch.empty(1, dtype=torch.int32, device=Qp.device)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=Qp.device)
    rc = _lib.load().bsa_build_mask(_ptr(Qp), _ptr(Kp), _DT[Qp.dtype], G, F, H, W, d,
                                    _ptr(axis_order), ctypes.byref(params), _ptr(row_ptr),
                                    _ptr(col_idx), col_idx.numel(), _ptr(nnz), _ptr(workspace),
                                    workspace.numel(), _stream())
    check(rc)
    return row_ptr, col_idx, nnz


def permute_pool(x, axis_order, F, H, W, B, out=None, sums=None, int8=None, reordered=True):
    """bsa_permute_pool: natural x [N][G][d] -> reordered bf16 [G][N][d] in one
    pass, also writing per-block channel sums and INT8 codes when asked.
    ``sums``: True (allocate) or an fp32 [G][ceil(N/B)][d] tensor, or None;
    ``int8``: True or a (codes int8 [G][N][d], scales fp32 [G][ceil(N/B)])
    pair, or None; ``reordered=False`` skips the bf16 copy.  Returns
    (xp or None, sums or None, (codes, scales) or None)."""
    _lib.load()
    N = F * H * W
    if x.dim() != 3 or x.shape[0] != N or x.stride(2) != 1:
        raise ValueError("natural input must be [N][G][d] with unit channel stride")
    G, d = x.shape[1], x.shape[2]
    nb = (N + B - 1) // B
    dev = x.device
    if not reordered:
        out = None
    elif out is None:
        out = torch.empty((G, N, d), dtype=torch.bfloat16, device=dev)
    if sums is True:
        sums = torch.empty((G, nb, d), dtype=torch.float32, device=dev)
    if int8 is True:
        int8 = (torch.empty((G, N, d), dtype=torch.int8, device=dev),
                torch.empty((G, nb), dtype=torch.float32, device=dev))
    xq, sc = int8 if int8 else (None, None)
    _dev(x, axis_order, *(t for t in (out, sums, xq, sc) if t is not None))
    if axis_order.dtype != torch.uint8 or axis_order.numel() < G:
        raise ValueError("axis_order must be a uint8 tensor with G entries")
    if out is not None and (out.shape != (G, N, d) or not out.is_contiguous()
                            or out.dtype != torch.bfloat16):
        raise ValueError("out must be contiguous bf16 [G][N][d]")
    if sums is not None and (sums.shape != (G, nb, d) or sums.dtype != torch.float32
                             or not sums.is_contiguous()):
        raise ValueError("sums must be contiguous fp32 [G][ceil(N/B)][d]")
    if xq is not None and (xq.shape != (G, N, d) or xq.dtype != torch.int8 or not xq.is_contiguous()
                           or sc.shape != (G, nb) or sc.dtype != torch.float32
                           or not sc.is_contiguous()):
        raise ValueError("int8 must be (int8 [G][N][d], fp32 [G][ceil(N/B)]), both contiguous")
    rc = _lib.load().bsa_permute_pool(
        _ptr(x), _DT[x.dtype], _ptr(out) if out is not None else None, x.stride(1), x.stride(0), G,
        F, H, W, d, _ptr(axis_order),
        B, _ptr(sums) if sums is not None else None, _ptr(xq) if xq is not None else None,
        _ptr(sc) if sc is not None else None, _stream())
    check(rc)
    return out, sums, (int8 if int8 else None)


def build_mask_pooled(sums_q, sums_k, axis_order, F, H, W, params: MaskParams, workspace=None):
    """bsa_build_mask_pooled from per-block channel sums (Bq blocks of the
    reordered Q, Bk blocks of the reordered K).  Returns (row_ptr, col_idx,
    nnz) as :func:`build_mask`."""
    _dev(sums_q, sums_k, axis_order)
    G, _, d = sums_q.shape
    N = F * H * W
    for t, B in ((sums_q, params.Bq), (sums_k, params.Bk)):
        if (t.shape != (G, (N + B - 1) // B, d) or t.dtype != torch.float32
                or not t.is_contiguous()):
            raise ValueError("sums must be contiguous fp32 [G][ceil(N/B)][d] (Bq for Q, Bk for K)")
    cap = mask_capacity(G, F, H, W, params)
    ws_bytes = mask_workspace(G, F, H, W, d, params)
    nq = (N + params.Bq - 1) // params.Bq
    row_ptr = torch.empty(G * nq + 1, dtype=torch.int32, device=sums_q.device)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=sums_q.device)
    nnz = torch.empty(1, dtype=torch.int32, device=sums_q.device)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=sums_q.device)
    rc = _lib.load().bsa_build_mask_pooled(_ptr(sums_q), _ptr(sums_k), G, F, H, W, d,
                                           _ptr(axis_order), ctypes.byref(params), _ptr(row_ptr),
                                           _ptr(col_idx), col_idx.numel(), _ptr(nnz),
                                           _ptr(workspace), workspace.numel(), _stream())
    check(rc)
    return row_ptr, col_idx, nnz


def build_mask_pooled_noalloc(sums_q, sums_k, axis_order, F, H, W, params: MaskParams, row_ptr,
                              col_idx, nnz):
    """bsa_build_mask_pooled_noalloc: as :func:`build_mask_pooled` into the
    caller's row_ptr (int32 [G*Nq+1]), col_idx (int32, >= mask_capacity) and
    nnz (int32 [1]), with the library's fixed device scratch in place of a
    workspace; neither this call nor the library allocates device memory."""
    G, _, d = sums_q.shape
    N = F * H * W
    for t, B in ((sums_q, params.Bq), (sums_k, params.Bk)):
        if (t.shape != (G, (N + B - 1) // B, d) or t.dtype != torch.float32
                or not t.is_contiguous()):
            raise ValueError("sums must be contiguous fp32 [G][ceil(N/B)][d] (Bq for Q, Bk for K)")
    nq = (N + params.Bq - 1) // params.Bq
    for name, t, n in (("row_ptr", row_ptr, G * nq + 1), ("nnz", nnz, 1), ("col_idx", col_idx, 0)):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() < n:
            raise ValueError(f"{name} must be contiguous int32 with at least {n} entries")
    _dev(sums_q, sums_k, axis_order, row_ptr, col_idx, nnz)
    check(_lib.load().bsa_build_mask_pooled_noalloc(
        _ptr(sums_q), _ptr(sums_k), G, F, H, W, d, _ptr(axis_order), ctypes.byref(params),
        _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _ptr(nnz), _stream()))
    return row_ptr, col_idx, nnz


def block_scores(sums_q, sums_k, F, H, W, params: MaskParams, out=None, workspace=None):
    """bsa_block_scores: fp32 [G][Nq][Nkv] scores of every (q-block, kv-block)
    pair from per-block channel sums (the keys the mask build ranks)."""
    _dev(sums_q, sums_k)
    G, _, d = sums_q.shape
    N = F * H * W
    nq, nk = (N + params.Bq - 1) // params.Bq, (N + params.Bk - 1) // params.Bk
    for t, nb in ((sums_q, nq), (sums_k, nk)):
        if t.shape != (G, nb, d) or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("sums must be contiguous fp32 [G][ceil(N/B)][d] (Bq for Q, Bk for K)")
    if out is None:
        out = torch.empty((G, nq, nk), dtype=torch.float32, device=sums_q.device)
    if out.shape != (G, nq, nk) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [G][Nq][Nkv]")
    ws_bytes = mask_workspace(G, F, H, W, d, params)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=sums_q.device)
    check(_lib.load().bsa_block_scores(_ptr(sums_q), _ptr(sums_k), G, F, H, W, d,
                                       ctypes.byref(params), _ptr(out), _ptr(workspace),
                                       workspace.numel(), _stream()))
    return out


def scores_select_workspace(G, F, H, W, Bq, Bk) -> int:
    v = int(_lib.load().bsa_scores_select_workspace(G, F, H, W, Bq, Bk))
    if v < 0:
        raise ValueError("bsa_scores_select_workspace: unsupported sizes")
    return v


def mask_from_scores(scores, axis_order, F, H, W, params: MaskParams, top_p=None, temp=1.0,
                     noise=None, noise_scale=1.0, workspace=None):
    """bsa_mask_from_scores: Top-K (top_p None: the budget of ``params``) or
    Top-P (top_p in (0, 1], weights exp2((score - max) * temp)) per q-block
    row of scores fp32 [G][Nq][Nkv], optionally perturbed by ``noise`` (same
    shape; score' = fma(noise, noise_scale, score)), plus the forced
    diagonal / window of ``params``.  Returns (row_ptr, col_idx, nnz) with
    col_idx the full-capacity buffer and nnz a device int32 [1]."""
    G, nq, nk = scores.shape
    N = F * H * W
    if nq != (N + params.Bq - 1) // params.Bq or nk != (N + params.Bk - 1) // params.Bk:
        raise ValueError("scores shape does not match the grid and blocks")
    for t in (scores, noise):
        if t is not None and (t.shape != scores.shape or t.dtype != torch.float32
                              or not t.is_contiguous()):
            raise ValueError("scores / noise must be contiguous fp32 [G][Nq][Nkv]")
    _dev(scores, axis_order, *(t for t in (noise,) if t is not None))
    mode = 0 if top_p is None else 1
    cap = mask_capacity(G, F, H, W, params) if mode == 0 else G * nq * nk
    ws_bytes = scores_select_workspace(G, F, H, W, params.Bq, params.Bk)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=scores.device)
    row_ptr = torch.empty(G * nq + 1, dtype=torch.int32, device=scores.device)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=scores.device)
    nnz = torch.empty(1, dtype=torch.int32, device=scores.device)
    check(_lib.load().bsa_mask_from_scores(_ptr(scores), _ptr(noise) if noise is not None else None,
                                           float(noise_scale), G, F, H, W, _ptr(axis_order),
                                           ctypes.byref(params), mode,
                                           float(top_p) if top_p is not None else 0.0, float(temp),
                                           _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _ptr(nnz),
                                           _ptr(workspace), workspace.numel(), _stream()))
    return row_ptr, col_idx, nnz


def order_workspace(G, F, H, W, B) -> int:
    v = int(_lib.load().bsa_order_workspace(G, F, H, W, B))
    if v < 0:
        raise ValueError("bsa_order_workspace: bad sizes or block")
    return v


def order_scores(x, F, H, W, B, out=None, workspace=None):
    """bsa_order_scores: SICS score of every (head, axis order) for natural
    x [N][G][d] (fp32 or bf16, unit channel stride) cut into B-row blocks.
    Returns fp32 [G][6] on the device."""
    _lib.load()
    N = F * H * W
    if x.dim() != 3 or x.shape[0] != N or x.stride(2) != 1:
        raise ValueError("natural input must be [N][G][d] with unit channel stride")
    G, d = x.shape[1], x.shape[2]
    if out is None:
        out = torch.empty((G, 6), dtype=torch.float32, device=x.device)
    if out.shape != (G, 6) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [G][6]")
    ws_bytes = order_workspace(G, F, H, W, B)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    _dev(x, out, workspace)
    rc = _lib.load().bsa_order_scores(_ptr(x), _DT[x.dtype], x.stride(1), x.stride(0), G, F, H, W, d,
                                      B, _ptr(out), _ptr(workspace), workspace.numel(), _stream())
    check(rc)
    return out


def select_orders(scores_a, scores_b=None, out=None):
    """bsa_select_orders: per head, the order code maximising
    scores_a + scores_b (fp32), ties to the lowest code.  Returns uint8 [G]."""
    G = scores_a.shape[0]
    for t in (scores_a, scores_b):
        if t is not None and (t.shape != (G, 6) or t.dtype != torch.float32
                              or not t.is_contiguous()):
            raise ValueError("scores must be contiguous fp32 [G][6]")
    if out is None:
        out = torch.empty(G, dtype=torch.uint8, device=scores_a.device)
    _dev(scores_a, out, *(t for t in (scores_b,) if t is not None))
    rc = _lib.load().bsa_select_orders(_ptr(scores_a), _ptr(scores_b) if scores_b is not None else None,
                                       G, _ptr(out), _stream())
    check(rc)
    return out


def attn_block_stats(Qp, Kp, B, eps=1e-3, sm_scale=0.0, out=None):
    """bsa_attn_block_stats: per-block statistics of the dense post-softmax
    map of reordered bf16 Qp, Kp [G][N][d].  Returns (cnt int32, bsum fp32,
    bmax fp32), each [G][nb][nb] with nb = ceil(N/B)."""
    _dev(Qp, Kp)
    G, N, d = Qp.shape
    if Kp.shape != Qp.shape or Qp.dtype != torch.bfloat16 or Kp.dtype != torch.bfloat16:
        raise ValueError("Qp and Kp must be bf16 [G][N][d] of one shape")
    if not (Qp.is_contiguous() and Kp.is_contiguous()):
        raise ValueError("Qp and Kp must be contiguous")
    nb = (N + B - 1) // B
    if out is None:
        out = (torch.empty((G, nb, nb), dtype=torch.int32, device=Qp.device),
               torch.empty((G, nb, nb), dtype=torch.float32, device=Qp.device),
               torch.empty((G, nb, nb), dtype=torch.float32, device=Qp.device))
    cnt, bsum, bmax = out
    for t, dt in ((cnt, torch.int32), (bsum, torch.float32), (bmax, torch.float32)):
        if t.shape != (G, nb, nb) or t.dtype != dt or not t.is_contiguous():
            raise ValueError("outputs must be contiguous [G][nb][nb] (int32, fp32, fp32)")
    _dev(cnt, bsum, bmax)
    check(_lib.load().bsa_attn_block_stats(_ptr(Qp), _ptr(Kp), G, N, d, B, float(sm_scale),
                                           float(eps), _ptr(cnt), _ptr(bsum), _ptr(bmax), _stream()))
    return cnt, bsum, bmax


def paro_metric(cnt, bsum, bmax, N, B, order, sigma=(9, 10), alpha=0.0, stats=None):
    """bsa_paro_metric: writes stats[g][order] = (M, r, Ibar) from one
    order's block statistics.  ``stats``: fp32 [G][6][3] (new if None)."""
    G = cnt.shape[0]
    if stats is None:
        stats = torch.full((G, 6, 3), float("nan"), dtype=torch.float32, device=cnt.device)
    if stats.shape != (G, 6, 3) or stats.dtype != torch.float32 or not stats.is_contiguous():
        raise ValueError("stats must be contiguous fp32 [G][6][3]")
    nb = (N + B - 1) // B
    for t in (cnt, bsum, bmax):
        if t.shape != (G, nb, nb) or not t.is_contiguous():
            raise ValueError("block statistics must be contiguous [G][nb][nb]")
    if cnt.dtype != torch.int32 or bsum.dtype != torch.float32 or bmax.dtype != torch.float32:
        raise ValueError("block statistics must be (int32, fp32, fp32)")
    _dev(cnt, bsum, bmax, stats)
    check(_lib.load().bsa_paro_metric(_ptr(cnt), _ptr(bsum), _ptr(bmax), G, N, B, int(sigma[0]),
                                      int(sigma[1]), float(alpha), int(order), _ptr(stats), _stream()))
    return stats


def paro_select(stats, out=None):
    """bsa_paro_select: per head, the order with the smallest M.  uint8 [G]."""
    G = stats.shape[0]
    if stats.shape != (G, 6, 3) or stats.dtype != torch.float32 or not stats.is_contiguous():
        raise ValueError("stats must be contiguous fp32 [G][6][3]")
    if out is None:
        out = torch.empty(G, dtype=torch.uint8, device=stats.device)
    _dev(stats, out)
    check(_lib.load().bsa_paro_select(_ptr(stats), G, _ptr(out), _stream()))
    return out


def paro_calibrate(Q, K, F, H, W, B=64, eps=1e-3, sigma=(9, 10), alpha=0.0, sm_scale=0.0):
    """Offline order choice for natural Q, K [N][G][d]: for each of the six
    axis orders, reorder (bsa_permute), take the dense map's block
    statistics and the order metric; then pick the argmin per head.
    Returns (axis_order uint8 [G], stats fp32 [G][6][3])."""
    G = Q.shape[1]
    stats = torch.full((G, 6, 3), float("nan"), dtype=torch.float32, device=Q.device)
    for o in range(6):
        orders = torch.full((G,), o, dtype=torch.uint8, device=Q.device)
        Qp = permute(Q, orders, F, H, W)
        Kp = permute(K, orders, F, H, W)
        cnt, bsum, bmax = attn_block_stats(Qp, Kp, B, eps, sm_scale)
        paro_metric(cnt, bsum, bmax, F * H * W, B, o, sigma, alpha, stats)
    return paro_select(stats), stats


def mask_from_block_sums(keys, N, Bq, Bk, mass, force_diag=True, workspace=None):
    """bsa_mask_from_block_sums: static mask keeping, per q-block row, the
    fewest largest blocks whose fp32 running sum reaches mass * row total
    (plus the diagonal).  keys fp32 [G][Nq][Nkv].  Returns (row_ptr, col_idx
    view of length nnz, nnz)."""
    G, nq, nk = keys.shape
    if keys.dtype != torch.float32 or not keys.is_contiguous():
        raise ValueError("keys must be contiguous fp32 [G][Nq][Nkv]")
    if nq != (N + Bq - 1) // Bq or nk != (N + Bk - 1) // Bk:
        raise ValueError("keys shape does not match N, Bq, Bk")
    ws = int(_lib.load().bsa_mask_sums_workspace(G, N, Bq, Bk))
    if ws < 0:
        raise ValueError("bsa_mask_sums_workspace: unsupported sizes")
    if workspace is None or workspace.numel() < ws:
        workspace = torch.empty(ws, dtype=torch.uint8, device=keys.device)
    row_ptr = torch.empty(G * nq + 1, dtype=torch.int32, device=keys.device)
    col_idx = torch.empty(G * nq * nk, dtype=torch.int32, device=keys.device)
    nnz = torch.empty(1, dtype=torch.int32, device=keys.device)
    _dev(keys, workspace)
    check(_lib.load().bsa_mask_from_block_sums(_ptr(keys), G, N, Bq, Bk, float(mass),
                                               1 if force_diag else 0, _ptr(row_ptr), _ptr(col_idx),
                                               col_idx.numel(), _ptr(nnz), _ptr(workspace),
                                               workspace.numel(), _stream()))
    n = int(nnz.item())
    return row_ptr, col_idx[:n], n


def mask_from_bits(bits, nk, workspace=None):
    """bsa_mask_from_bits: CSR of a block bitmask, bits int64/uint64
    [rows][ceil(nk/64)] (bit j % 64 of word j // 64 keeps kv-block j).
    Returns (row_ptr, col_idx view of length nnz, nnz)."""
    rows, words = bits.shape
    if words != (nk + 63) // 64 or bits.element_size() != 8 or not bits.is_contiguous():
        raise ValueError("bits must be contiguous 64-bit [rows][ceil(nk/64)]")
    ws = int(_lib.load().bsa_mask_bits_workspace(rows))
    if workspace is None or workspace.numel() < ws:
        workspace = torch.empty(ws, dtype=torch.uint8, device=bits.device)
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=bits.device)
    col_idx = torch.empty(rows * nk, dtype=torch.int32, device=bits.device)
    nnz = torch.empty(1, dtype=torch.int32, device=bits.device)
    _dev(bits, workspace)
    check(_lib.load().bsa_mask_from_bits(_ptr(bits), rows, nk, _ptr(row_ptr), _ptr(col_idx),
                                         col_idx.numel(), _ptr(nnz), _ptr(workspace),
                                         workspace.numel(), _stream()))
    n = int(nnz.item())
    return row_ptr, col_idx[:n], n


def quantize_int8(Xp, B, out=None):
    """bsa_quantize_int8: bf16 [G][N][d] -> (int8 [G][N][d], fp32 scales
    [G][ceil(N/B)]); ``out`` = (q, scale) reuses preallocated tensors."""
    if Xp.dim() != 3 or Xp.dtype != torch.bfloat16 or not Xp.is_contiguous():
        raise ValueError("Xp must be contiguous bf16 [G][N][d]")
    G, N, d = Xp.shape
    if out is not None:
        q, s = out
        if (q.dtype != torch.int8 or tuple(q.shape) != (G, N, d) or not q.is_contiguous()
                or s.dtype != torch.float32 or not s.is_contiguous() or s.numel() < G * -(-N // B)):
            raise ValueError("out must be (int8 [G][N][d], fp32 [G][ceil(N/B)]), contiguous")
    _dev(Xp, *(out or ()))
    if out is None:
        q = torch.empty((G, N, d), dtype=torch.int8, device=Xp.device)
        s = torch.empty((G, (N + B - 1) // B), dtype=torch.float32, device=Xp.device)
    else:
        q, s = out
    check(_lib.load().bsa_quantize_int8(_ptr(Xp), _ptr(q), _ptr(s), G, N, d, B, _stream()))
    return q, s


def _attn_inputs(Q, K, V, row_ptr, col_idx, Bq, Bk, mask_G, col_len, dtype, scales=None):
    """Host checks of a forward's inputs that the C ABI cannot make (it sees
    raw pointers): shapes, dtypes, contiguity and lengths, so that no kernel
    reads past an allocation.  Returns (G, N, d, mask_G, col_len)."""
    if Q.dim() != 3:
        raise ValueError("Q must be [G][N][d]")
    G, N, d = Q.shape
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}")
        if tuple(t.shape) != (G, N, d):
            raise ValueError(f"{name} must have Q's shape {(G, N, d)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [G][N][d]")
    if Bq not in (64, 128) or Bk not in (64, 128):
        raise ValueError("Bq and Bk must be 64 or 128")
    nq, nk = -(-N // Bq), -(-N // Bk)
    mask_G = G if mask_G is None else int(mask_G)
    if not 1 <= mask_G <= G:
        raise ValueError("mask_G must be in [1, G]")
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 1-D int32 tensor")
    if row_ptr.numel() < mask_G * nq + 1:
        raise ValueError(f"row_ptr needs mask_G*Nq + 1 = {mask_G * nq + 1} entries "
                         f"(Bq = {Bq}), got {row_ptr.numel()}")
    col_len = col_idx.numel() if col_len is None else int(col_len)
    if not 0 <= col_len <= col_idx.numel():
        raise ValueError("col_len must be in [0, col_idx.numel()]")
    if scales is not None:
        for name, t, n in zip(("sQ", "sK", "sV"), scales, (G * nq, G * nk, G * nk)):
            if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() < n:
                raise ValueError(f"{name} must be contiguous fp32 with at least {n} entries")
    return G, N, d, mask_G, col_len


def _check_lse(lse, G, N):
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.numel() != G * N):
        raise ValueError("lse must be contiguous fp32 with G*N entries")


def _lse_out(lse, want_lse, G, N, dev):
    if lse is None and want_lse:
        lse = torch.empty((G, N), dtype=torch.float32, device=dev)
    return lse


def _check_reordered_out(out, G, N, d):
    if out is not None and (tuple(out.shape) != (G, N, d) or out.dtype != torch.bfloat16
                            or not out.is_contiguous()):
        raise ValueError("out must be contiguous bf16 [G][N][d]")


def _reordered_out(out, G, N, d, dev):
    if out is None:
        out = torch.empty((G, N, d), dtype=torch.bfloat16, device=dev)
    return out


def forward(Qp, Kp, Vp, row_ptr, col_idx, Bq, Bk, mask_G=None, sm_scale=0.0, out=None,
            lse=None, want_lse=True, col_len=None):
    """bsa_forward: bf16 block-sparse attention on reordered tensors.
    Returns (O bf16 [G][N][d], lse fp32 [G][N] or None)."""
    G, N, d, mask_G, col_len = _attn_inputs(Qp, Kp, Vp, row_ptr, col_idx, Bq, Bk, mask_G, col_len,
                                            torch.bfloat16)
    _check_reordered_out(out, G, N, d)
    _check_lse(lse, G, N)
    _dev(Qp, Kp, Vp, row_ptr, col_idx, out, lse)
    out = _reordered_out(out, G, N, d, Qp.device)
    lse = _lse_out(lse, want_lse, G, N, Qp.device)
    rc = _lib.load().bsa_forward(_ptr(Qp), _ptr(Kp), _ptr(Vp), _ptr(row_ptr), _ptr(col_idx),
                                 col_len, mask_G, _ptr(out), _ptr(lse), G, N, d, Bq, Bk,
                                 float(sm_scale), _stream())
    check(rc)
    return out, lse


def forward_int8(Qq, sQ, Kq, sK, Vq, sV, row_ptr, col_idx, Bq, Bk, mask_G=None, sm_scale=0.0,
                 out=None, lse=None, want_lse=True, col_len=None):
    """bsa_forward_int8 on int8 reordered tensors with per-block scales."""
    G, N, d, mask_G, col_len = _attn_inputs(Qq, Kq, Vq, row_ptr, col_idx, Bq, Bk, mask_G, col_len,
                                            torch.int8, (sQ, sK, sV))
    _check_reordered_out(out, G, N, d)
    _check_lse(lse, G, N)
    _dev(Qq, sQ, Kq, sK, Vq, sV, row_ptr, col_idx, out, lse)
    out = _reordered_out(out, G, N, d, Qq.device)
    lse = _lse_out(lse, want_lse, G, N, Qq.device)
    rc = _lib.load().bsa_forward_int8(_ptr(Qq), _ptr(sQ), _ptr(Kq), _ptr(sK), _ptr(Vq), _ptr(sV),
                                      _ptr(row_ptr), _ptr(col_idx), col_len, mask_G, _ptr(out),
                                      _ptr(lse), G, N, d, Bq, Bk, float(sm_scale), _stream())
    check(rc)
    return out, lse


def _orders_ok(axis_order, G):
    if axis_order.dtype != torch.uint8 or axis_order.numel() < G:
        raise ValueError("axis_order must be a uint8 tensor with G entries")


def _check_natural_out(out, G, N, d):
    if out is not None and (out.dim() != 3 or out.shape != (N, G, d) or out.stride(2) != 1
                            or out.dtype != torch.bfloat16):
        raise ValueError("out must be bf16 [N][G][d] (any strides with unit channel stride)")


def _natural_out(out, G, N, d, dev):
    if out is None:
        out = torch.empty((N, G, d), dtype=torch.bfloat16, device=dev)
    return out


def forward_natural(Qp, Kp, Vp, row_ptr, col_idx, Bq, Bk, axis_order, F, H, W, mask_G=None,
                    sm_scale=0.0, out=None, lse=None, want_lse=True, col_len=None):
    """bsa_forward_natural: bsa_forward with the inverse reorder fused into
    its epilogue.  Returns (O bf16 natural [N][G][d] (``out`` may be a
    strided view), lse fp32 [G][N] by natural token or None)."""
    G, N, d, mask_G, col_len = _attn_inputs(Qp, Kp, Vp, row_ptr, col_idx, Bq, Bk, mask_G, col_len,
                                            torch.bfloat16)
    if N != F * H * W:
        raise ValueError("N must equal F*H*W")
    _orders_ok(axis_order, G)
    _check_natural_out(out, G, N, d)
    _check_lse(lse, G, N)
    _dev(Qp, Kp, Vp, row_ptr, col_idx, axis_order, out, lse)
    out = _natural_out(out, G, N, d, Qp.device)
    lse = _lse_out(lse, want_lse, G, N, Qp.device)
    rc = _lib.load().bsa_forward_natural(_ptr(Qp), _ptr(Kp), _ptr(Vp), _ptr(row_ptr), _ptr(col_idx),
                                         col_len, mask_G, _ptr(axis_order), F, H, W, _ptr(out),
                                         out.stride(1), out.stride(0), _ptr(lse), G, d, Bq, Bk,
                                         float(sm_scale), _stream())
    check(rc)
    return out, lse


def forward_int8_natural(Qq, sQ, Kq, sK, Vq, sV, row_ptr, col_idx, Bq, Bk, axis_order, F, H, W,
                         mask_G=None, sm_scale=0.0, out=None, lse=None, want_lse=True,
                         col_len=None):
    """bsa_forward_int8_natural: bsa_forward_int8 writing O in natural order."""
    G, N, d, mask_G, col_len = _attn_inputs(Qq, Kq, Vq, row_ptr, col_idx, Bq, Bk, mask_G, col_len,
                                            torch.int8, (sQ, sK, sV))
    if N != F * H * W:
        raise ValueError("N must equal F*H*W")
    _orders_ok(axis_order, G)
    _check_natural_out(out, G, N, d)
    _check_lse(lse, G, N)
    _dev(Qq, sQ, Kq, sK, Vq, sV, row_ptr, col_idx, axis_order, out, lse)
    out = _natural_out(out, G, N, d, Qq.device)
    lse = _lse_out(lse, want_lse, G, N, Qq.device)
    rc = _lib.load().bsa_forward_int8_natural(
        _ptr(Qq), _ptr(sQ), _ptr(Kq), _ptr(sK), _ptr(Vq), _ptr(sV), _ptr(row_ptr), _ptr(col_idx),
        col_len, mask_G, _ptr(axis_order), F, H, W, _ptr(out), out.stride(1), out.stride(0),
        _ptr(lse), G, d, Bq, Bk, float(sm_scale), _stream())
    check(rc)
    return out, lse


def fo_workspace(G, N, d, Bq, Bk) -> int:
    v = int(_lib.load().bsa_fo_workspace(G, N, d, Bq, Bk))
    if v < 0:
        check(v)
    return v


def fo_compensate(Qp, Kp, Vp, row_ptr, col_idx, Bq, Bk, O, lse, axis_order=None, F=None, H=None,
                  W=None, mask_G=None, sm_scale=0.0, workspace=None, col_len=None):
    """bsa_fo_compensate: adds the first-order compensation of each q-block
    row's skipped keys to a forward's output, in place.  ``O``, ``lse`` as
    :func:`forward` wrote them (``axis_order`` None: reordered [G][N][d] and
    [G][N]) or as :func:`forward_natural` did (``axis_order`` given: natural
    [N][G][d], any strides with unit channel stride, lse by natural token).
    Returns (O, lse)."""
    G, N, d, mask_G, col_len = _attn_inputs(Qp, Kp, Vp, row_ptr, col_idx, Bq, Bk, mask_G, col_len,
                                            torch.bfloat16)
    if F is None:
        F, H, W = 1, 1, N
    if F * H * W != N:
        raise ValueError("N must equal F*H*W")
    if lse is None:
        raise ValueError("lse is required")
    _check_lse(lse, G, N)
    if axis_order is None:
        _check_reordered_out(O, G, N, d)
        sg, sn = 0, 0
    else:
        _orders_ok(axis_order, G)
        _check_natural_out(O, G, N, d)
        sg, sn = O.stride(1), O.stride(0)
    need = fo_workspace(G, N, d, Bq, Bk)
    _dev(Qp, Kp, Vp, row_ptr, col_idx, O, lse, axis_order, workspace)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=Qp.device)
    check(_lib.load().bsa_fo_compensate(
        _ptr(Qp), _ptr(Kp), _ptr(Vp), _ptr(row_ptr), _ptr(col_idx), col_len, mask_G,
        _ptr(axis_order), F, H, W, _ptr(O), sg, sn, _ptr(lse), G, d, Bq, Bk, float(sm_scale),
        _ptr(workspace), workspace.numel(), _stream()))
    return O, lse


def debug_int8_qk(Qq, Kq, gij, Bq, Bk):
    """bsa_debug_int8_qk: exact int32 Q.K^T tiles for gij int32 [n][3] of (g, i, j)."""
    _dev(Qq, Kq, gij)
    G, N, d = Qq.shape
    n = gij.shape[0]
    S = torch.empty((n, Bq, Bk), dtype=torch.int32, device=Qq.device)
    check(_lib.load().bsa_debug_int8_qk(_ptr(Qq), _ptr(Kq), G, N, d, Bq, Bk, _ptr(gij), n, _ptr(S),
                                        _stream()))
    return S


def debug_int8_pv(P8, Vq, gj, Bq, Bk):
    """bsa_debug_int8_pv: exact int32 P.V tiles, P8 int8 [n][Bq][Bk], gj int32 [n][2]."""
    _dev(P8, Vq, gj)
    G, N, d = Vq.shape
    n = gj.shape[0]
    OV = torch.empty((n, Bq, d), dtype=torch.int32, device=Vq.device)
    check(_lib.load().bsa_debug_int8_pv(_ptr(P8), _ptr(Vq), G, N, d, Bq, Bk, _ptr(gj), n, _ptr(OV),
                                        _stream()))
    return OV


class LayerPlan:
    """Buffers for one attention layer over natural-order [N][G][d] tensors:
    reordered copies, mask CSR, INT8 copies and the output, allocated once
    and reused by :func:`layer_forward`.  ``compensate=True`` adds the
    first-order compensation of the skipped keys after the forward (its
    workspace allocated here; it reads the bf16 reordered Q, K, V, which the
    INT8 chain then also writes)."""

    def __init__(self, G, F, H, W, d, device, params: MaskParams, int8=False, dynamic_mask=True,
                 fused=False, compensate=False):
        N = F * H * W
        self.G, self.F, self.H, self.W, self.d, self.N = G, F, H, W, d, N
        self.params = params
        self.int8 = int8
        self.dynamic_mask = dynamic_mask
        self.fused = fused
        self.compensate = compensate
        e = dict(device=device)
        self.Qp = torch.empty((G, N, d), dtype=torch.bfloat16, **e)
        self.Kp = torch.empty_like(self.Qp)
        self.Vp = torch.empty_like(self.Qp)
        self.Op = torch.empty_like(self.Qp)
        self.lse = torch.empty((G, N), dtype=torch.float32, **e)
        self.O = torch.empty((N, G, d), dtype=torch.bfloat16, **e)
        nq = (N + params.Bq - 1) // params.Bq
        cap = mask_capacity(G, F, H, W, params)
        self.row_ptr = torch.zeros(G * nq + 1, dtype=torch.int32, **e)
        self.col_idx = torch.zeros(max(cap, 1), dtype=torch.int32, **e)
        self.nnz = torch.zeros(1, dtype=torch.int32, **e)
        self.ws = torch.empty(mask_workspace(G, F, H, W, d, params), dtype=torch.uint8, **e)
        if fused:
            nk = (N + params.Bk - 1) // params.Bk
            self.sums_q = torch.empty((G, nq, d), dtype=torch.float32, **e)
            self.sums_k = torch.empty((G, nk, d), dtype=torch.float32, **e)
        if compensate:
            self.fo_ws = torch.empty(fo_workspace(G, N, d, params.Bq, params.Bk), dtype=torch.uint8,
                                     **e)
        if int8:
            nk = (N + params.Bk - 1) // params.Bk
            self.Qq = torch.empty((G, N, d), dtype=torch.int8, **e)
            self.Kq = torch.empty_like(self.Qq)
            self.Vq = torch.empty_like(self.Qq)
            self.sQ = torch.empty((G, nq), dtype=torch.float32, **e)
            self.sK = torch.empty((G, nk), dtype=torch.float32, **e)
            self.sV = torch.empty((G, nk), dtype=torch.float32, **e)

    def quantize(self):
        p = self.params
        quantize_int8(self.Qp, p.Bq, out=(self.Qq, self.sQ))
        quantize_int8(self.Kp, p.Bk, out=(self.Kq, self.sK))
        quantize_int8(self.Vp, p.Bk, out=(self.Vq, self.sV))

    def reorder_fused(self, Q, K, V, axis_order):
        """Reorder Q, K, V with the block sums of Q and K (and, for INT8, the
        codes of all three) in the same pass."""
        p = self.params
        q8 = (self.Qq, self.sQ) if self.int8 else None
        k8 = (self.Kq, self.sK) if self.int8 else None
        v8 = (self.Vq, self.sV) if self.int8 else None
        F, H, W = self.F, self.H, self.W
        # the INT8 attention reads only the codes; the compensation reads bf16
        bf = not self.int8 or self.compensate
        permute_pool(Q, axis_order, F, H, W, p.Bq, out=self.Qp, sums=self.sums_q, int8=q8,
                     reordered=bf)
        permute_pool(K, axis_order, F, H, W, p.Bk, out=self.Kp, sums=self.sums_k, int8=k8,
                     reordered=bf)
        if self.int8:
            permute_pool(V, axis_order, F, H, W, p.Bk, out=self.Vp, int8=v8, reordered=bf)
        else:
            permute_pool(V, axis_order, F, H, W, p.Bk, out=self.Vp)

    def build_mask_from_sums(self, axis_order):
        lib = _lib.load()
        check(lib.bsa_build_mask_pooled(_ptr(self.sums_q), _ptr(self.sums_k), self.G, self.F,
                                        self.H, self.W, self.d, _ptr(axis_order),
                                        ctypes.byref(self.params), _ptr(self.row_ptr),
                                        _ptr(self.col_idx), self.col_idx.numel(), _ptr(self.nnz),
                                        _ptr(self.ws), self.ws.numel(), _stream()))

    def build_mask(self, axis_order):
        lib = _lib.load()
        p = self.params
        check(lib.bsa_build_mask(_ptr(self.Qp), _ptr(self.Kp), BSA_BF16, self.G, self.F, self.H,
                                 self.W, self.d, _ptr(axis_order), ctypes.byref(p),
                                 _ptr(self.row_ptr), _ptr(self.col_idx), self.col_idx.numel(),
                                 _ptr(self.nnz), _ptr(self.ws), self.ws.numel(), _stream()))


def layer_forward(plan: LayerPlan, Q, K, V, axis_order):
    """One pass of the whole path on natural-order Q, K, V [N][G][d]:
    reorder (x3) -> [build mask] -> [quantize (x3)] -> block-sparse attention
    -> inverse reorder.  With ``plan.fused`` the reorder, the block pooling
    and the INT8 quantisation share one pass per tensor, and the inverse
    reorder is the attention's own epilogue (``plan.lse`` is then indexed by
    natural token).  With ``plan.compensate`` the first-order compensation
    of the skipped keys follows the attention.  Returns the natural-order
    output [N][G][d] (bf16)."""
    F, H, W = plan.F, plan.H, plan.W
    p = plan.params
    if plan.fused:
        plan.reorder_fused(Q, K, V, axis_order)
        if plan.dynamic_mask:
            plan.build_mask_from_sums(axis_order)
    else:
        permute(Q, axis_order, F, H, W, 0, out=plan.Qp)
        permute(K, axis_order, F, H, W, 0, out=plan.Kp)
        permute(V, axis_order, F, H, W, 0, out=plan.Vp)
        if plan.dynamic_mask:
            plan.build_mask(axis_order)
        if plan.int8:
            plan.quantize()
    if plan.fused:
        if plan.int8:
            forward_int8_natural(plan.Qq, plan.sQ, plan.Kq, plan.sK, plan.Vq, plan.sV, plan.row_ptr,
                                 plan.col_idx, p.Bq, p.Bk, axis_order, F, H, W, out=plan.O,
                                 lse=plan.lse)
        else:
            forward_natural(plan.Qp, plan.Kp, plan.Vp, plan.row_ptr, plan.col_idx, p.Bq, p.Bk,
                            axis_order, F, H, W, out=plan.O, lse=plan.lse)
        if plan.compensate:
            fo_compensate(plan.Qp, plan.Kp, plan.Vp, plan.row_ptr, plan.col_idx, p.Bq, p.Bk, plan.O,
                          plan.lse, axis_order, F, H, W, workspace=plan.fo_ws)
        return plan.O
    if plan.int8:
        forward_int8(plan.Qq, plan.sQ, plan.Kq, plan.sK, plan.Vq, plan.sV, plan.row_ptr,
                     plan.col_idx, p.Bq, p.Bk, out=plan.Op, lse=plan.lse)
    else:
        forward(plan.Qp, plan.Kp, plan.Vp, plan.row_ptr, plan.col_idx, p.Bq, p.Bk, out=plan.Op,
                lse=plan.lse)
    if plan.compensate:
        fo_compensate(plan.Qp, plan.Kp, plan.Vp, plan.row_ptr, plan.col_idx, p.Bq, p.Bk, plan.Op,
                      plan.lse, F=F, H=H, W=W, workspace=plan.fo_ws)
    permute(plan.Op, axis_order, F, H, W, 1, out=plan.O)
    return plan.O
