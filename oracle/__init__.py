"""CPU oracle for the block-sparse video attention path.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
(``block_sparse_attention_inverse_amd``) never imports it, and this package
never imports the product.  All arrays are host numpy arrays.

The arithmetic lives in ``bsa_oracle.c`` (plain C, fp64 for attention, a
fixed fp32 sequence for block scoring and INT8 quantisation); this module
only marshals arguments.  ``brute.py`` holds pure-Python cross-checks for
tiny inputs.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, I8, F64 = 0, 1, 2, 3

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_D = ctypes.c_double


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "oracle_perm": (_I, [_I, _I, _I, _I, _P]),
        "oracle_f32_to_bf16": (None, [_P, _P, _L]),
        "oracle_permute": (_I, [_I, _P, _I, _P, _I, _L, _L, _I, _I, _I, _I, _I, _P]),
        "oracle_block_sums": (_I, [_P, _I, _L, _I, _I, _P]),
        "oracle_block_keys": (_I, [_P, _P, _L, _L, _I, _I, _I, _L, _I, _P]),
        "oracle_select_k": (_L, [_L, _I, _I]),
        "oracle_select": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _I, _I, _I, _I, _I, _P, _P, _L, _P]),
        "oracle_build_mask": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                   _P, _P, _L, _P, _P]),
        "oracle_quantize_int8": (_I, [_P, _I, _L, _I, _I, _P, _P]),
        "oracle_attention_rows": (_I, [_P, _P, _P, _I, _L, _L, _I, _I, _I, _I, _I, _P, _I, _I, _P,
                                       _P, _I, _I, _D, _P, _L, _P, _P]),
        "oracle_attention_int8": (_I, [_P, _P, _P, _P, _P, _P, _I, _L, _I, _I, _I, _P, _P, _I, _D,
                                       _I, _P, _L, _P, _P]),
        "oracle_int8_qk_tile": (_I, [_P, _P, _I, _L, _I, _I, _I, _L, _L, _P]),
        "oracle_int8_pv_tile": (_I, [_P, _P, _I, _L, _I, _I, _I, _L, _P]),
        "oracle_sics_scores": (_I, [_P, _I, _L, _L, _I, _I, _I, _I, _I, _I, _P]),
        "oracle_block_stats": (_I, [_P, _P, _I, _L, _I, _I, _D, _D, _D, _P, _P, _P, _P, _P]),
        "oracle_block_stats_rows": (_I, [_P, _P, _I, _L, _I, _I, _D, _D, _D, _P, _L, _P, _P, _P,
                                         _P, _P]),
        "oracle_paro_metric": (_I, [_P, _P, _P, _I, _L, _I, _I, _I, _D, _P]),
        "oracle_mass_select": (_I, [_P, _I, _L, _I, _I, ctypes.c_float, _I, _P, _P, _L, _P]),
        "oracle_exp2_fixed": (ctypes.c_float, [ctypes.c_float]),
        "oracle_attention_rows_fo": (_I, [_P, _P, _P, _I, _L, _L, _I, _I, _I, _I, _I, _P, _I, _I,
                                          _P, _P, _I, _D, _P, _L, _P, _P]),
        "oracle_perturb_keys": (None, [_P, _P, ctypes.c_float, _L, _P]),
        "oracle_select_topp": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, ctypes.c_float, ctypes.c_float,
                                    _I, _I, _I, _P, _P, _L, _P, _P, _P]),
        "oracle_num_threads": (_I, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # bf16 bit patterns
        return BF16
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.int8:
        return I8
    raise TypeError(f"unsupported dtype {a.dtype}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def perm(order: int, F: int, H: int, W: int) -> np.ndarray:
    """perm[p] = natural index of reordered position p (PAROAttention token reordering)."""
    out = np.empty(F * H * W, dtype=np.int32)
    _check(_load().oracle_perm(int(order), F, H, W, _ptr(out)), "perm")
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_f32_to_bf16(_ptr(x), _ptr(y), x.size)
    return y


def bf16_to_f64(x: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def permute(direction, src, dst_dtype, G, F, H, W, d, orders, stride_g=None, stride_n=None,
            natural_shape=None):
    """Gather (0: natural -> reordered [G][N][d]) or scatter (1: reordered -> natural).

    The natural side is [N][G][d] by default (stride_n = G*d, stride_g = d).
    ``src``/result use uint16 for bf16 bit patterns and float32 for fp32.
    """
    N = F * H * W
    if stride_g is None:
        stride_g, stride_n = d, G * d
    src = np.ascontiguousarray(src)
    orders = np.ascontiguousarray(orders, dtype=np.uint8)
    if direction == 0:
        dst = np.empty((G, N, d), dtype=dst_dtype)
    else:
        shape = natural_shape if natural_shape is not None else (N, G, d)
        dst = np.zeros(shape, dtype=dst_dtype)
    rc = _load().oracle_permute(direction, _ptr(src), _dtype_code(src), _ptr(dst), _dtype_code(dst),
                                stride_g, stride_n, G, F, H, W, d, _ptr(orders))
    _check(rc, "permute")
    return dst


def block_sums(Xp: np.ndarray, B: int) -> np.ndarray:
    G, N, d = Xp.shape
    Xp = np.ascontiguousarray(Xp, dtype=np.uint16)
    nb = (N + B - 1) // B
    S = np.empty((G, nb, d), dtype=np.float32)
    _check(_load().oracle_block_sums(_ptr(Xp), G, N, d, B, _ptr(S)), "block_sums")
    return S


def block_keys(Sq: np.ndarray, Sk: np.ndarray, N: int, Bq: int, Bk: int, score: int) -> np.ndarray:
    """fp32 keys of one head: Sq [nq][d], Sk [nk][d] -> [nq][nk]."""
    Sq = np.ascontiguousarray(Sq, dtype=np.float32)
    Sk = np.ascontiguousarray(Sk, dtype=np.float32)
    nq, d = Sq.shape
    nk = Sk.shape[0]
    key = np.empty((nq, nk), dtype=np.float32)
    _check(_load().oracle_block_keys(_ptr(Sq), _ptr(Sk), nq, nk, d, Bq, Bk, N, score, _ptr(key)),
           "block_keys")
    return key


def select_k(nk: int, rho_num: int, rho_den: int) -> int:
    return int(_load().oracle_select_k(nk, rho_num, rho_den))


def select(keys, G, F, H, W, Bq, Bk, orders, rho_num, rho_den, force_diag, win_T, win_r0):
    """CSR (row_ptr, col_idx) from per-head keys [G][nq][nk]."""
    keys = np.ascontiguousarray(keys, dtype=np.float32)
    orders = np.ascontiguousarray(orders, dtype=np.uint8)
    N = F * H * W
    nq, nk = (N + Bq - 1) // Bq, (N + Bk - 1) // Bk
    cap = G * nq * nk
    row_ptr = np.empty(G * nq + 1, dtype=np.int32)
    col_idx = np.empty(max(cap, 1), dtype=np.int32)
    nnz = ctypes.c_int64(0)
    rc = _load().oracle_select(_ptr(keys), G, F, H, W, Bq, Bk, _ptr(orders), rho_num, rho_den,
                               force_diag, win_T, win_r0, _ptr(row_ptr), _ptr(col_idx), cap,
                               ctypes.byref(nnz))
    _check(rc, "select")
    return row_ptr, col_idx[: nnz.value].copy()


def build_mask(Qp, Kp, F, H, W, orders, Bq, Bk, score, rho_num, rho_den, force_diag=1,
               win_T=-1, win_r0=0, audit=False):
    """Whole mask build (sums -> keys -> select) from reordered bf16 Qp, Kp [G][N][d].

    Returns (row_ptr, col_idx) or, with audit=True, (row_ptr, col_idx, near_ties).
    """
    Qp = np.ascontiguousarray(Qp, dtype=np.uint16)
    Kp = np.ascontiguousarray(Kp, dtype=np.uint16)
    orders = np.ascontiguousarray(orders, dtype=np.uint8)
    G, N, d = Qp.shape
    nq, nk = (N + Bq - 1) // Bq, (N + Bk - 1) // Bk
    cap = G * nq * nk
    row_ptr = np.empty(G * nq + 1, dtype=np.int32)
    col_idx = np.empty(max(cap, 1), dtype=np.int32)
    nnz = ctypes.c_int64(0)
    ties = ctypes.c_int64(0)
    rc = _load().oracle_build_mask(_ptr(Qp), _ptr(Kp), G, F, H, W, d, _ptr(orders), Bq, Bk, score,
                                   rho_num, rho_den, force_diag, win_T, win_r0, _ptr(row_ptr),
                                   _ptr(col_idx), cap, ctypes.byref(nnz),
                                   ctypes.byref(ties) if audit else None)
    _check(rc, "build_mask")
    out = (row_ptr, col_idx[: nnz.value].copy())
    return out + (ties.value,) if audit else out


def quantize_int8(Xp: np.ndarray, B: int):
    """Per-(head, block) symmetric INT8: returns (q int8 [G][N][d], scale fp32 [G][nb])."""
    Xp = np.ascontiguousarray(Xp, dtype=np.uint16)
    G, N, d = Xp.shape
    nb = (N + B - 1) // B
    q = np.empty((G, N, d), dtype=np.int8)
    s = np.empty((G, nb), dtype=np.float32)
    _check(_load().oracle_quantize_int8(_ptr(Xp), G, N, d, B, _ptr(q), _ptr(s)), "quantize_int8")
    return q, s


def sics_scores(X, G, F, H, W, d, B, stride_g=None, stride_n=None):
    """SPADE's online blocking score for each (head, PARO axis order): the
    fp32 closed-form sum of intra-block cosine similarities, [G][6] fp32.
    X: natural-order fp32 or bf16 (uint16) array, default [N][G][d]."""
    if stride_g is None:
        stride_g, stride_n = d, G * d
    X = np.ascontiguousarray(X)
    out = np.empty((G, 6), dtype=np.float32)
    _check(_load().oracle_sics_scores(_ptr(X), _dtype_code(X), stride_g, stride_n, G, F, H, W, d,
                                      B, _ptr(out)), "sics_scores")
    return out


def select_orders(scores_a, scores_b=None):
    """Per head, the order code with the largest fp32 scores_a + scores_b;
    ties go to the lowest code (numpy's argmax returns the first maximum)."""
    s = np.asarray(scores_a, dtype=np.float32)
    if scores_b is not None:
        s = s + np.asarray(scores_b, dtype=np.float32)
    return np.argmax(s, axis=1).astype(np.uint8)


def attention_rows(Q, K, V, G, F, H, W, d, orders, rows, Bq=64, Bk=64, row_ptr=None,
                   col_idx=None, mask_G=None, dense=False, sm_scale=None, stride_g=None,
                   stride_n=None):
    """fp64 masked softmax attention for natural-order rows.

    Q, K, V: natural-order arrays (float32, float64, or uint16 bf16 bits) with
    element (n, g, c) at n*stride_n + g*stride_g + c (default [N][G][d]).
    rows: int array [R][2] of (g, n).  Returns (O [R][d] fp64, lse [R] fp64).
    """
    Q, K, V = (np.ascontiguousarray(x) for x in (Q, K, V))
    assert Q.dtype == K.dtype == V.dtype
    if stride_g is None:
        stride_g, stride_n = d, G * d
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
    orders = np.ascontiguousarray(orders, dtype=np.uint8)
    R = rows.shape[0]
    O = np.zeros((R, d), dtype=np.float64)
    lse = np.zeros(R, dtype=np.float64)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    if not dense:
        row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
        col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
        if mask_G is None:
            mask_G = G
    rc = _load().oracle_attention_rows(
        _ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), stride_g, stride_n, G, F, H, W, d,
        _ptr(orders), Bq, Bk, None if dense else _ptr(row_ptr), None if dense else _ptr(col_idx),
        0 if dense else mask_G, 1 if dense else 0, float(sm_scale), _ptr(rows), R, _ptr(O),
        _ptr(lse))
    _check(rc, "attention_rows")
    return O, lse


def attention_rows_fo(Q, K, V, G, F, H, W, d, orders, rows, Bq, Bk, row_ptr, col_idx,
                      mask_G=None, sm_scale=None, stride_g=None, stride_n=None):
    """fp64 masked attention plus the first-order compensation of each
    q-block row's skipped keys (one expansion point, their mean), for
    natural-order rows; arguments as :func:`attention_rows` (mask required).
    Returns (O [R][d], lse [R])."""
    Q, K, V = (np.ascontiguousarray(x) for x in (Q, K, V))
    assert Q.dtype == K.dtype == V.dtype
    if stride_g is None:
        stride_g, stride_n = d, G * d
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
    orders = np.ascontiguousarray(orders, dtype=np.uint8)
    R = rows.shape[0]
    O = np.zeros((R, d), dtype=np.float64)
    lse = np.zeros(R, dtype=np.float64)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
    rc = _load().oracle_attention_rows_fo(
        _ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), stride_g, stride_n, G, F, H, W, d,
        _ptr(orders), Bq, Bk, _ptr(row_ptr), _ptr(col_idx), G if mask_G is None else mask_G,
        float(sm_scale), _ptr(rows), R, _ptr(O), _ptr(lse))
    _check(rc, "attention_rows_fo")
    return O, lse


def attention_int8(Qq, sQ, Kq, sK, Vq, sV, Bq, Bk, row_ptr, col_idx, blocks, mask_G=None,
                   sm_scale=None, quantize_p=True):
    """Online-order INT8 attention for reordered q-blocks.

    Qq/Kq/Vq int8 [G][N][d]; sQ fp32 [G][nq]; sK, sV fp32 [G][nk].
    blocks: int array [B][2] of (g, i).  Returns (O [B][Bq][d], lse [B][Bq]) fp64.
    """
    Qq, Kq, Vq = (np.ascontiguousarray(x, dtype=np.int8) for x in (Qq, Kq, Vq))
    sQ, sK, sV = (np.ascontiguousarray(x, dtype=np.float32) for x in (sQ, sK, sV))
    G, N, d = Qq.shape
    blocks = np.ascontiguousarray(blocks, dtype=np.int64).reshape(-1, 2)
    nb = blocks.shape[0]
    O = np.zeros((nb, Bq, d), dtype=np.float64)
    lse = np.zeros((nb, Bq), dtype=np.float64)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    if mask_G is None:
        mask_G = G
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
    rc = _load().oracle_attention_int8(
        _ptr(Qq), _ptr(sQ), _ptr(Kq), _ptr(sK), _ptr(Vq), _ptr(sV), G, N, d, Bq, Bk,
        _ptr(row_ptr), _ptr(col_idx), mask_G, float(sm_scale), 1 if quantize_p else 0,
        _ptr(blocks), nb, _ptr(O), _ptr(lse))
    _check(rc, "attention_int8")
    return O, lse


def int8_qk_tile(Qq, Kq, g, i, j, Bq, Bk):
    Qq, Kq = np.ascontiguousarray(Qq, np.int8), np.ascontiguousarray(Kq, np.int8)
    G, N, d = Qq.shape
    S = np.empty((Bq, Bk), dtype=np.int32)
    _check(_load().oracle_int8_qk_tile(_ptr(Qq), _ptr(Kq), g, N, d, Bq, Bk, i, j, _ptr(S)), "qk")
    return S


def int8_pv_tile(P8, Vq, g, j, Bq, Bk):
    P8, Vq = np.ascontiguousarray(P8, np.int8), np.ascontiguousarray(Vq, np.int8)
    G, N, d = Vq.shape
    OV = np.empty((Bq, d), dtype=np.int32)
    _check(_load().oracle_int8_pv_tile(_ptr(P8), _ptr(Vq), g, N, d, Bq, Bk, j, _ptr(OV)), "pv")
    return OV


def block_stats(Qp, Kp, B, eps, sm_scale=None, delta=1e-3):
    """Block statistics of the dense fp64 post-softmax map of reordered bf16
    Qp, Kp [G][N][d] (PAROAttention calibration): dict of cnt (entries
    below eps), cnt_lo / cnt_hi (below eps*(1 -/+ delta)), sum, max, each
    [G][nb][nb]."""
    Qp = np.ascontiguousarray(Qp, dtype=np.uint16)
    Kp = np.ascontiguousarray(Kp, dtype=np.uint16)
    G, N, d = Qp.shape
    nb = (N + B - 1) // B
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = {k: np.empty((G, nb, nb), dtype=np.int32) for k in ("cnt", "cnt_lo", "cnt_hi")}
    out["sum"] = np.empty((G, nb, nb), dtype=np.float64)
    out["max"] = np.empty((G, nb, nb), dtype=np.float64)
    _check(_load().oracle_block_stats(_ptr(Qp), _ptr(Kp), G, N, d, B, float(sm_scale), float(eps),
                                      float(delta), _ptr(out["cnt"]), _ptr(out["cnt_lo"]),
                                      _ptr(out["cnt_hi"]), _ptr(out["sum"]), _ptr(out["max"])),
           "block_stats")
    return out


def perturb_keys(keys, noise, scale):
    """Seeded stochastic scoring: key' = fmaf(noise, scale, key) in fp32
    (noise None: key unchanged); the random draws come in as ``noise``."""
    keys = np.ascontiguousarray(keys, dtype=np.float32)
    out = np.empty_like(keys)
    nz = None if noise is None else np.ascontiguousarray(noise, dtype=np.float32)
    _load().oracle_perturb_keys(_ptr(keys), _ptr(nz), ctypes.c_float(scale), keys.size, _ptr(out))
    return out


def exp2_fixed(a: float) -> float:
    """The fixed fp32 2^a that defines the Top-P weights (one fp32 value)."""
    return float(_load().oracle_exp2_fixed(float(np.float32(a))))


def select_topp(keys, G, F, H, W, Bq, Bk, orders, top_p, temp, force_diag=1, win_T=-1, win_r0=0):
    """Top-P selection on fp32 keys [G][nq][nk]: returns (row_ptr, col_idx,
    kstar [G*nq], cum [G*nq][nk] fp64 running weights in sorted order)."""
    keys = np.ascontiguousarray(keys, dtype=np.float32)
    orders = np.ascontiguousarray(orders, dtype=np.uint8)
    nq, nk = keys.shape[1], keys.shape[2]
    row_ptr = np.empty(G * nq + 1, dtype=np.int32)
    cap = G * nq * nk
    col_idx = np.empty(cap, dtype=np.int32)
    kstar = np.empty(G * nq, dtype=np.int32)
    cum = np.empty((G * nq, nk), dtype=np.float64)
    nnz = ctypes.c_int64(0)
    _check(_load().oracle_select_topp(_ptr(keys), G, F, H, W, Bq, Bk, _ptr(orders),
                                      ctypes.c_float(top_p), ctypes.c_float(temp), force_diag, win_T,
                                      win_r0, _ptr(row_ptr), _ptr(col_idx), cap, ctypes.byref(nnz),
                                      _ptr(kstar), _ptr(cum)), "select_topp")
    return row_ptr, col_idx[: nnz.value].copy(), kstar, cum


def block_stats_rows(Qp, Kp, B, eps, blocks, sm_scale=None, delta=1e-3):
    """block_stats for chosen (head, q-block) rows only: blocks int [n][2]
    of (g, i); returns the same dict with arrays [n][nb]."""
    Qp = np.ascontiguousarray(Qp, dtype=np.uint16)
    Kp = np.ascontiguousarray(Kp, dtype=np.uint16)
    G, N, d = Qp.shape
    nb = (N + B - 1) // B
    blocks = np.ascontiguousarray(blocks, dtype=np.int64)
    n = blocks.shape[0]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = {k: np.empty((n, nb), dtype=np.int32) for k in ("cnt", "cnt_lo", "cnt_hi")}
    out["sum"] = np.empty((n, nb), dtype=np.float64)
    out["max"] = np.empty((n, nb), dtype=np.float64)
    _check(_load().oracle_block_stats_rows(_ptr(Qp), _ptr(Kp), G, N, d, B, float(sm_scale),
                                           float(eps), float(delta), _ptr(blocks), n,
                                           _ptr(out["cnt"]), _ptr(out["cnt_lo"]),
                                           _ptr(out["cnt_hi"]), _ptr(out["sum"]),
                                           _ptr(out["max"])), "block_stats_rows")
    return out


def paro_metric(cnt, bsum, bmax, N, B, sigma_num, sigma_den, alpha):
    """Per head (M, r, Ibar) in fp64 from one order's block statistics
    (cnt int32, sum and max fp32, [G][nb][nb]): r = share of sparse blocks,
    Ibar = mean block incoherence, M = (1 - r) + alpha*Ibar."""
    cnt = np.ascontiguousarray(cnt, dtype=np.int32)
    bsum = np.ascontiguousarray(bsum, dtype=np.float32)
    bmax = np.ascontiguousarray(bmax, dtype=np.float32)
    G = cnt.shape[0]
    out = np.empty((G, 3), dtype=np.float64)
    _check(_load().oracle_paro_metric(_ptr(cnt), _ptr(bsum), _ptr(bmax), G, N, B, sigma_num,
                                      sigma_den, float(alpha), _ptr(out)), "paro_metric")
    return out


def paro_select(metric):
    """Per head, the order code with the smallest M (metric [G][6]); ties go
    to the lowest code."""
    return np.argmin(np.asarray(metric), axis=1).astype(np.uint8)


def mass_select(keys, N, Bq, Bk, mass, force_diag=1):
    """Static mask by block-sum thresholding: keys fp32 [G][nq][nk] (block
    sums); returns (row_ptr, col_idx) int32."""
    keys = np.ascontiguousarray(keys, dtype=np.float32)
    G, nq, nk = keys.shape
    row_ptr = np.empty(G * nq + 1, dtype=np.int32)
    cap = G * nq * nk
    col_idx = np.empty(max(cap, 1), dtype=np.int32)
    nnz = ctypes.c_int64(0)
    _check(_load().oracle_mass_select(_ptr(keys), G, N, Bq, Bk, ctypes.c_float(mass), force_diag,
                                      _ptr(row_ptr), _ptr(col_idx), cap, ctypes.byref(nnz)),
           "mass_select")
    return row_ptr, col_idx[: nnz.value].copy()


def bits_to_csr(bits, nk):
    """CSR of a block bitmask: bits uint64 [R][words], bit j % 64 of word
    j // 64 set keeps kv-block j; bits at j >= nk are ignored.  The kept
    indices of each row in ascending order."""
    bits = np.asarray(bits, dtype=np.uint64)
    R = bits.shape[0]
    row_ptr = np.zeros(R + 1, dtype=np.int32)
    cols = []
    for r in range(R):
        row = [j for j in range(nk) if (int(bits[r, j // 64]) >> (j % 64)) & 1]
        cols.extend(row)
        row_ptr[r + 1] = row_ptr[r] + len(row)
    return row_ptr, np.asarray(cols, dtype=np.int32)
