"""The C ABI library: it loads, exports every entry point the header
declares (and no undeclared bsa_* symbol), and its host-side checks answer
without touching a GPU.  No compute call is made here."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(bsa_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from block_sparse_attention_inverse_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_attention_inverse_amd import build

        build.build()
    return _lib.load()


def test_header_lists_the_entry_points():
    names = header_functions()
    for n in ("bsa_permute", "bsa_build_mask", "bsa_forward", "bsa_forward_int8",
              "bsa_quantize_int8", "bsa_mask_capacity", "bsa_mask_workspace",
              "bsa_debug_int8_qk", "bsa_debug_int8_pv", "bsa_abi_version", "bsa_last_error",
              "bsa_permute_pool", "bsa_build_mask_pooled", "bsa_order_workspace",
              "bsa_order_scores", "bsa_select_orders", "bsa_attn_block_stats",
              "bsa_paro_metric", "bsa_paro_select", "bsa_mask_sums_workspace",
              "bsa_mask_from_block_sums", "bsa_mask_bits_workspace", "bsa_mask_from_bits",
              "bsa_block_scores", "bsa_scores_select_workspace", "bsa_mask_from_scores",
              "bsa_forward_natural", "bsa_forward_int8_natural"):
        assert n in names


def test_exports_match_header(lib):
    from block_sparse_attention_inverse_amd import _lib

    names = header_functions()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_lib.SIGNATURES) == names
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if re.search(r" T bsa_", l)})
    assert exported == names


def test_version_and_error_text(lib):
    assert lib.bsa_abi_version() == 1
    assert lib.bsa_last_error() in (b"", None) or isinstance(lib.bsa_last_error(), bytes)


def test_mask_capacity_and_workspace_host_only(lib):
    from block_sparse_attention_inverse_amd._lib import MaskParams

    p = MaskParams(128, 64, 0, 30, 100, 1, -1, 0)
    cap = lib.bsa_mask_capacity(40, 21, 45, 80, ctypes.byref(p))
    nq, nk = -(-75600 // 128), -(-75600 // 64)
    assert cap == 40 * nq * (355 + 3)
    ws = lib.bsa_mask_workspace(40, 21, 45, 80, 128, ctypes.byref(p))
    assert ws >= 4 * 40 * (nq + nk) * 128
    pw = MaskParams(128, 128, 1, 15, 100, 1, 2, 4)
    assert lib.bsa_mask_capacity(24, 33, 45, 80, ctypes.byref(pw)) == 24 * 929 * 929
    bad = MaskParams(96, 64, 0, 30, 100, 1, -1, 0)
    assert lib.bsa_mask_capacity(1, 4, 8, 8, ctypes.byref(bad)) == -2
    assert b"64 or 128" in lib.bsa_last_error()
    bad2 = MaskParams(64, 64, 0, 30, 0, 1, -1, 0)
    assert lib.bsa_mask_capacity(1, 4, 8, 8, ctypes.byref(bad2)) == -1
    assert lib.bsa_mask_capacity(1, 4, 8, 8, None) == -1


def test_argument_errors_before_any_launch(lib):
    """Rejected calls return an error code and a message; none reaches HIP."""
    P = ctypes.c_void_p
    fake = P(0x1000)
    # NULL tensors
    assert lib.bsa_forward(None, None, None, None, None, 0, 1, None, None, 1, 64, 128, 128, 64,
                           0.0, None) == -1
    # unsupported head dim
    assert lib.bsa_forward(fake, fake, fake, fake, fake, 10, 1, fake, None, 1, 64, 96, 128, 64,
                           0.0, None) == -2
    assert b"d must be 64 or 128" in lib.bsa_last_error()
    # misaligned pointer
    assert lib.bsa_forward(P(0x1001), fake, fake, fake, fake, 10, 1, fake, None, 1, 64, 128, 128,
                           64, 0.0, None) == -1
    # bad mask_G
    assert lib.bsa_forward(fake, fake, fake, fake, fake, 10, 3, fake, None, 2, 64, 128, 128, 64,
                           0.0, None) == -1
    # permute: bad direction, bad d, bad dtype
    assert lib.bsa_permute(2, fake, 1, fake, 1, 8, 8, 1, 1, 1, 8, 8, fake, None) == -1
    assert lib.bsa_permute(0, fake, 1, fake, 1, 8, 8, 1, 1, 1, 8, 12, fake, None) == -1
    assert lib.bsa_permute(0, fake, 2, fake, 1, 8, 8, 1, 1, 1, 8, 8, fake, None) == -2
    # quantize: bad block
    assert lib.bsa_quantize_int8(fake, fake, fake, 1, 64, 64, 32, None) == -2
    # build_mask: capacity too small
    from block_sparse_attention_inverse_amd._lib import MaskParams

    p = MaskParams(64, 64, 0, 30, 100, 1, -1, 0)
    assert lib.bsa_build_mask(fake, fake, 1, 1, 4, 8, 8, 64, fake, ctypes.byref(p), fake, fake, 1,
                              fake, P(0x1000), 1 << 20, None) == -3
    assert b"col_capacity" in lib.bsa_last_error()
    assert lib.bsa_build_mask(fake, fake, 0, 1, 4, 8, 8, 64, fake, ctypes.byref(p), fake, fake,
                              1 << 20, fake, P(0x1000), 1 << 20, None) == -2


def test_fused_and_order_argument_errors(lib):
    """Host checks of the fused pass, the pooled mask build and the order
    scores; none of these calls reaches HIP."""
    P = ctypes.c_void_p
    fake = P(0x1000)
    # permute_pool: no output at all, xq without scale, bad B, misaligned dst
    assert lib.bsa_permute_pool(fake, 1, None, 8, 64, 1, 2, 4, 8, 64, fake, 64, None, None, None,
                                None) == -1
    assert b"no output" in lib.bsa_last_error()
    assert lib.bsa_permute_pool(fake, 1, fake, 8, 64, 1, 2, 4, 8, 64, fake, 64, None, fake, None,
                                None) == -1
    assert lib.bsa_permute_pool(fake, 1, fake, 8, 64, 1, 2, 4, 8, 64, fake, 32, None, None, None,
                                None) == -2
    assert lib.bsa_permute_pool(fake, 1, P(0x1008), 8, 64, 1, 2, 4, 8, 64, fake, 64, None, None,
                                None, None) == -1
    # build_mask_pooled: capacity too small
    from block_sparse_attention_inverse_amd._lib import MaskParams

    p = MaskParams(64, 64, 0, 30, 100, 1, -1, 0)
    assert lib.bsa_build_mask_pooled(fake, fake, 1, 4, 8, 8, 64, fake, ctypes.byref(p), fake, fake,
                                     1, fake, P(0x1000), 1 << 20, None) == -3
    # order scores: workspace size and a short workspace
    assert lib.bsa_order_workspace(40, 21, 45, 80, 128) == -(-4 * 40 * 6 * 591 // 256) * 256 + 4 * 40 * 75600
    assert lib.bsa_order_workspace(1, 2, 3, 4, 96) == -1
    assert lib.bsa_order_scores(fake, 1, 8, 64, 1, 2, 4, 8, 64, 64, fake, fake, 4, None) == -3
    assert b"workspace" in lib.bsa_last_error()
    assert lib.bsa_order_scores(fake, 2, 8, 64, 1, 2, 4, 8, 64, 64, fake, fake, 1 << 20, None) == -2
    assert lib.bsa_select_orders(None, None, 4, fake, None) == -1


def test_calibration_and_static_mask_argument_errors(lib):
    """Host checks of the offline calibration and static-mask calls; none of
    these reaches HIP."""
    P = ctypes.c_void_p
    fake = P(0x1000)
    F = ctypes.c_float
    # block stats: bad d, bad B, non-positive eps, misaligned Q
    assert lib.bsa_attn_block_stats(fake, fake, 1, 256, 96, 64, F(0), F(1e-3), fake, fake, fake,
                                    None) == -2
    assert lib.bsa_attn_block_stats(fake, fake, 1, 256, 128, 32, F(0), F(1e-3), fake, fake, fake,
                                    None) == -2
    assert lib.bsa_attn_block_stats(fake, fake, 1, 256, 128, 64, F(0), F(0), fake, fake, fake,
                                    None) == -1
    assert b"eps" in lib.bsa_last_error()
    assert lib.bsa_attn_block_stats(P(0x1008), fake, 1, 256, 128, 64, F(0), F(1e-3), fake, fake,
                                    fake, None) == -1
    # metric: sigma out of range, order out of range, negative alpha
    assert lib.bsa_paro_metric(fake, fake, fake, 1, 256, 64, 11, 10, F(0), 0, fake, None) == -1
    assert lib.bsa_paro_metric(fake, fake, fake, 1, 256, 64, 9, 10, F(0), 6, fake, None) == -1
    assert lib.bsa_paro_metric(fake, fake, fake, 1, 256, 64, 9, 10, F(-1), 0, fake, None) == -1
    assert lib.bsa_paro_select(None, 4, fake, None) == -1
    # static mask from block sums: workspace size, mass range, capacity, workspace short
    ws = lib.bsa_mask_sums_workspace(2, 1000, 64, 64)
    R, nk = 2 * 16, 16
    assert ws == R * 1 * 8 + ((R * 4 + 255) // 256) * 256
    assert lib.bsa_mask_sums_workspace(2, 1000, 64, 96) == -1
    args = (fake, 2, 1000, 64, 64)
    assert lib.bsa_mask_from_block_sums(*args, F(0.0), 1, fake, fake, R * nk, fake, P(0x1000), ws,
                                        None) == -1
    assert lib.bsa_mask_from_block_sums(*args, F(1.5), 1, fake, fake, R * nk, fake, P(0x1000), ws,
                                        None) == -1
    assert lib.bsa_mask_from_block_sums(*args, F(0.9), 1, fake, fake, R * nk - 1, fake,
                                        P(0x1000), ws, None) == -3
    assert b"col_capacity" in lib.bsa_last_error()
    assert lib.bsa_mask_from_block_sums(*args, F(0.9), 1, fake, fake, R * nk, fake, P(0x1000),
                                        ws - 1, None) == -3
    # bitmask -> CSR: workspace size, capacity, alignment
    assert lib.bsa_mask_bits_workspace(10) == 256
    assert lib.bsa_mask_bits_workspace(0) == -1
    assert lib.bsa_mask_from_bits(fake, 10, 100, fake, fake, 999, fake, fake, 256, None) == -3
    assert lib.bsa_mask_from_bits(P(0x1004), 10, 100, fake, fake, 1000, fake, fake, 256,
                                  None) == -1


def test_scores_selection_argument_errors(lib):
    """Host checks of the score-matrix selection; none reaches HIP."""
    from block_sparse_attention_inverse_amd._lib import MaskParams

    P = ctypes.c_void_p
    fake = P(0x1000)
    F = ctypes.c_float
    p = MaskParams(64, 64, 0, 30, 100, 1, -1, 0)
    pw = MaskParams(64, 64, 0, 30, 100, 1, 2, 4)  # with a temporal window
    ws = lib.bsa_scores_select_workspace(2, 2, 8, 40, 64, 64)
    assert ws > 0 and lib.bsa_scores_select_workspace(2, 2, 8, 40, 64, 96) == -1
    big = 1 << 30
    args = (fake, None, F(0), 2, 2, 8, 40)
    # bad mode, top_p out of range, negative temperature, window without orders
    assert lib.bsa_mask_from_scores(*args, fake, ctypes.byref(p), 2, F(0.5), F(1), fake, fake, big,
                                    fake, P(0x1000), ws, None) == -1
    assert lib.bsa_mask_from_scores(*args, fake, ctypes.byref(p), 1, F(0.0), F(1), fake, fake, big,
                                    fake, P(0x1000), ws, None) == -1
    assert lib.bsa_mask_from_scores(*args, fake, ctypes.byref(p), 1, F(0.5), F(-1), fake, fake, big,
                                    fake, P(0x1000), ws, None) == -1
    assert lib.bsa_mask_from_scores(*args, None, ctypes.byref(pw), 0, F(0), F(0), fake, fake, big,
                                    fake, P(0x1000), ws, None) == -1
    assert b"axis_order" in lib.bsa_last_error()
    # capacity: top-p needs G*Nq*Nkv; a short workspace
    assert lib.bsa_mask_from_scores(*args, fake, ctypes.byref(p), 1, F(0.5), F(1), fake, fake,
                                    2 * 10 * 10 - 1, fake, P(0x1000), ws, None) == -3
    assert lib.bsa_mask_from_scores(*args, fake, ctypes.byref(p), 0, F(0), F(0), fake, fake, big,
                                    fake, P(0x1000), ws - 1, None) == -3
    # block scores: bad d, short workspace
    assert lib.bsa_block_scores(fake, fake, 2, 2, 8, 40, 96, ctypes.byref(p), fake, P(0x1000), big,
                                None) == -2
    assert lib.bsa_block_scores(fake, fake, 2, 2, 8, 40, 64, ctypes.byref(p), fake, P(0x1000), 16,
                                None) == -3


def test_forward_natural_argument_errors(lib):
    """Host checks of the forwards that write natural order; none reaches HIP."""
    P = ctypes.c_void_p
    fake = P(0x1000)
    F = ctypes.c_float
    G, d = 4, 128
    Fr, Hr, Wr = 2, 8, 40
    N = Fr * Hr * Wr
    ok = (d, G * d)  # [N][G][d]
    def call(orders=fake, grid=(Fr, Hr, Wr), strides=ok):
        return lib.bsa_forward_natural(fake, fake, fake, fake, fake, 100, G, orders, *grid, fake,
                                       strides[0], strides[1], None, G, d, 128, 64, F(0), None)
    assert call(orders=None) == -1
    assert call(grid=(0, Hr, Wr)) == -1
    assert call(strides=(d, d)) == -1            # rows of different heads overlap
    assert b"overlap" in lib.bsa_last_error()
    assert call(strides=(d + 4, G * (d + 4))) == -1  # not a multiple of 8
    assert lib.bsa_forward_int8_natural(fake, fake, fake, fake, fake, fake, fake, fake, 100, G, None,
                                        Fr, Hr, Wr, fake, d, G * d, None, G, d, 128, 64, F(0),
                                        None) == -1


def test_product_path_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """With libbsa.so absent the binding raises; nothing falls back to a CPU
    or PyTorch implementation."""
    from block_sparse_attention_inverse_amd import _lib
    import block_sparse_attention_inverse_amd as bsa

    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libbsa.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()
    with pytest.raises(ImportError):
        bsa.abi_version()
    with pytest.raises(ImportError):
        bsa.mask_capacity(1, 2, 8, 8, bsa.mask_params())


def test_forward_rejects_heads_too_long_for_32_bit_addressing(lib):
    """One head's K / V is addressed through 32-bit buffer resources: a head
    of 2^31 bytes or more is refused before any launch (bf16: N*d*2, INT8:
    N*d)."""
    P = ctypes.c_void_p
    fake = P(0x1000)
    F = ctypes.c_float
    N = 1 << 23  # N*128*2 = 2^31 bytes per bf16 head
    assert lib.bsa_forward(fake, fake, fake, fake, fake, 10, 1, fake, None, 1, N, 128, 128, 64,
                           F(0), None) == -2
    assert b"2^31 bytes" in lib.bsa_last_error()
    assert lib.bsa_forward_int8(fake, fake, fake, fake, fake, fake, fake, fake, 10, 1, fake, None, 1,
                                2 * N, 128, 128, 64, F(0), None) == -2
    assert b"2^31 bytes" in lib.bsa_last_error()
    # natural-order output: the same limit with N = F*H*W
    assert lib.bsa_forward_natural(fake, fake, fake, fake, fake, 10, 1, fake, 8, 1024, 1024, fake,
                                   128, 128, None, 1, 128, 128, 64, F(0), None) == -2


def test_forward_bindings_check_inputs_before_any_launch():
    """The Python forwards refuse inputs the C ABI cannot see through raw
    pointers (mismatched shapes, dtypes, strides, short row_ptr or scales)
    with ValueError, before any device check or launch."""
    import torch
    import block_sparse_attention_inverse_amd as bsa

    G, N, d, B = 2, 256, 64, 64
    nq = N // B
    Q = torch.zeros((G, N, d), dtype=torch.bfloat16)
    rp = torch.zeros(G * nq + 1, dtype=torch.int32)
    ci = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="shape"):
        bsa.forward(Q, Q[:, :128], Q, rp, ci, B, B)
    with pytest.raises(ValueError, match="bfloat16"):
        bsa.forward(Q, Q.float(), Q, rp, ci, B, B)
    with pytest.raises(ValueError, match="contiguous"):
        bsa.forward(Q, Q, Q.transpose(0, 1).contiguous().transpose(0, 1), rp, ci, B, B)
    with pytest.raises(ValueError, match="row_ptr needs"):
        bsa.forward(Q, Q, Q, rp[:nq], ci, B, B)
    with pytest.raises(ValueError, match="row_ptr needs"):  # a mask built with Bq = 128
        bsa.forward(Q, Q, Q, torch.zeros(G * N // 128 + 1, dtype=torch.int32), ci, B, B)
    with pytest.raises(ValueError, match="int32"):
        bsa.forward(Q, Q, Q, rp.long(), ci, B, B)
    with pytest.raises(ValueError, match="col_len"):
        bsa.forward(Q, Q, Q, rp, ci, B, B, col_len=5)
    with pytest.raises(ValueError, match="mask_G"):
        bsa.forward(Q, Q, Q, rp, ci, B, B, mask_G=3)
    with pytest.raises(ValueError, match="out must be"):
        bsa.forward(Q, Q, Q, rp, ci, B, B, out=torch.zeros((G, N, d + 8), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        bsa.forward(Q, Q, Q, rp, ci, B, B)
    q8 = torch.zeros((G, N, d), dtype=torch.int8)
    s = torch.zeros(G * nq, dtype=torch.float32)
    with pytest.raises(ValueError, match="sK must be"):
        bsa.forward_int8(q8, s, q8, s[:1], q8, s, rp, ci, B, B)
    with pytest.raises(ValueError, match="int8"):
        bsa.forward_int8(q8, s, Q, s, q8, s, rp, ci, B, B)
    with pytest.raises(ValueError, match="GPU"):
        bsa.forward_int8(q8, s, q8, s, q8, s, rp, ci, B, B)
    orders = torch.zeros(G, dtype=torch.uint8)
    with pytest.raises(ValueError, match="F\\*H\\*W"):
        bsa.forward_natural(Q, Q, Q, rp, ci, B, B, orders, 2, 2, 2)
    with pytest.raises(ValueError, match="axis_order"):
        bsa.forward_natural(Q, Q, Q, rp, ci, B, B, orders[:1], 4, 8, 8)
    with pytest.raises(ValueError, match="Xp must be"):
        bsa.quantize_int8(Q.float(), B)


def test_noalloc_mask_refuses_shapes_beyond_its_scratch(lib):
    """The mask build without allocation has a fixed 48 MiB scratch: a shape
    whose workspace exceeds it is refused (ECAPACITY, nothing launched), with
    a message naming both sizes."""
    from block_sparse_attention_inverse_amd._lib import MaskParams

    P = ctypes.c_void_p
    fake = P(0x1000)
    p = MaskParams(64, 64, 0, 30, 100, 1, -1, 0)  # 720p, 40 heads, 64x64: 53.6 MiB
    need = lib.bsa_mask_workspace(40, 21, 45, 80, 128, ctypes.byref(p))
    assert need > 48 << 20
    cap = lib.bsa_mask_capacity(40, 21, 45, 80, ctypes.byref(p))
    assert lib.bsa_build_mask_pooled_noalloc(fake, fake, 40, 21, 45, 80, 128, fake, ctypes.byref(p),
                                             fake, fake, cap, fake, None) == -3
    msg = lib.bsa_last_error()
    assert b"scratch" in msg and str(need).encode() in msg and b"50331648" in msg
    assert lib.bsa_build_mask_pooled_noalloc(None, fake, 40, 21, 45, 80, 128, fake, ctypes.byref(p),
                                             fake, fake, cap, fake, None) == -1


def test_compensation_argument_errors(lib):
    """Host checks of the first-order compensation; none reaches HIP."""
    P = ctypes.c_void_p
    fake = P(0x1000)
    F = ctypes.c_float
    G, d, Fr, Hr, Wr = 2, 128, 1, 4, 64
    N = Fr * Hr * Wr
    need = lib.bsa_fo_workspace(G, N, d, 128, 64)
    assert need > 0
    assert lib.bsa_fo_workspace(G, N, 96, 128, 64) == -2
    # the skip mask is addressed with 32-bit buffer ranges: Nq and Nkv at most 32768
    assert lib.bsa_fo_workspace(1, 32768 * 64, 64, 64, 64) > 0
    assert lib.bsa_fo_workspace(1, 32768 * 64 + 1, 64, 64, 128) == -2
    assert b"Nq" in lib.bsa_last_error()
    assert lib.bsa_fo_workspace(1, 32768 * 64 + 1, 64, 128, 64) == -2
    assert b"Nkv" in lib.bsa_last_error()
    def call(lse=fake, ws_bytes=need, ws=fake, orders=None):
        return lib.bsa_fo_compensate(fake, fake, fake, fake, fake, 10, G, orders, Fr, Hr, Wr, fake,
                                     d, G * d, lse, G, d, 128, 64, F(0), ws, ws_bytes, None)
    assert call(lse=None) == -1
    assert b"lse is required" in lib.bsa_last_error()
    assert call(ws_bytes=need - 1) == -3
    assert call(ws=P(0x1010)) == -1  # not 256-byte aligned
    assert call(orders=fake, ws_bytes=need - 1) == -3
