"""Benchmark of the block-sparse video attention path on one MI355X.

One step = one pass of the bf16 layer chain over one synthetic batch:
reorder Q, K, V (with the Q/K block sums in the same pass) -> build the
block mask (pooled DOT scores, per-row top-k, diagonal) -> bf16 block-sparse
flash attention whose epilogue writes O in natural token order (the inverse
reorder fused into it).
The INT8 chain (reorder with quantisation -> mask -> INT8 attention writing
natural order) is timed in the same run, over the same number of steps,
and reported under "int8"; the long-clip layer (118,800 tokens, mask rebuilt
every step from COSINE block scores with a temporal window) under
"long_clip"; the offline order calibration (dense-map block statistics for
all six axis orders, metric, argmin, static mask) under "calibration".

Workload: the 720p-shaped DiT layer, F=21, H=45, W=80 (75,600 tokens),
40 heads, d=128, 128x64 blocks, 30% density; inputs resident in HBM.

value = dense-equivalent attention TFLOPS = 4*N^2*d*G / (time per step).
roofline: the dominant kernel (bf16 attention) against the bf16 MFMA peak,
achieved = kept-block FLOPs per launch / its mean launch time, measured with
HIP events on the launch stream inside the timed region.
cpu_baseline: the CPU oracle on one head's share, extrapolated to the layer.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_INT8_TOPS = 5000.0  # MI355X dense int8 MFMA
METRIC = "dense-equiv attention TFLOPS + MFMA util at 30% density, 75.6k tokens"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_720p_traffic.txt")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kept_flops(row_ptr, col_idx, G, N, Bq, Bk, d):
    import numpy as np

    nq = (N + Bq - 1) // Bq
    counts = np.diff(row_ptr.astype(np.int64))
    rows_real = np.minimum(Bq, N - np.arange(nq) * Bq)
    rows_per_entry = np.repeat(np.tile(rows_real, G), counts)
    cols_real = np.minimum(Bk, N - col_idx.astype(np.int64) * Bk)
    return 4.0 * d * float(np.sum(rows_per_entry * cols_real))


ATTN_SOURCES = ("attn_bf16.hip", "bsa_device.hpp")
COPY_BYTES = 1 << 31  # plain device copy used to calibrate the HBM byte counters


def source_hash():
    """Hash of the bf16 attention kernel's sources with comments and blank
    lines dropped: a traffic figure taken on other code is stale and is not
    reported (an edit to comments alone keeps it)."""
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_attention_inverse_amd", "csrc", name)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def read_traffic(flops_per_launch):
    """Bytes per launch of the bf16 attention kernel beyond its L2 (FETCH_SIZE
    + WRITE_SIZE, copy-calibrated) from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("attn_source_sha256_16") != source_hash():
        return None
    try:
        return float(kv["l2_miss_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    """The host CPU's model string from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, Qn, Kn, Vn, orders, p, budget_s=12.0):
    """Oracle on head 0 (reorder, mask build, masked attention on sampled
    rows), extrapolated to the whole layer (all heads, all rows)."""
    import numpy as np

    import oracle
    from block_sparse_attention_inverse_amd import synth

    F, H, W, d, N, G = cfg["F"], cfg["H"], cfg["W"], cfg["d"], cfg["N"], cfg["G"]
    q, k, v = (synth.bf16_bits(x[:, :1, :]) for x in (Qn, Kn, Vn))
    o1 = orders[:1]
    t0 = time.perf_counter()
    qp = oracle.permute(0, q, np.uint16, 1, F, H, W, d, o1)
    kp = oracle.permute(0, k, np.uint16, 1, F, H, W, d, o1)
    vp = oracle.permute(0, v, np.uint16, 1, F, H, W, d, o1)
    rp, ci = oracle.build_mask(qp, kp, F, H, W, o1, p.Bq, p.Bk, p.score, p.rho_num, p.rho_den,
                               p.force_diag, p.win_T, p.win_r0)
    t_head = time.perf_counter() - t0
    r = np.random.Generator(np.random.PCG64(7))
    probe = np.stack([np.zeros(64, np.int64), r.integers(0, N, 64)], axis=1)
    t0 = time.perf_counter()
    oracle.attention_rows(q, k, v, 1, F, H, W, d, o1, probe, p.Bq, p.Bk, rp, ci)
    t_probe = time.perf_counter() - t0
    nrows = int(max(64, min(N, (budget_s - t_head) / max(t_probe / 64, 1e-6))))
    rows = np.stack([np.zeros(nrows, np.int64), r.integers(0, N, nrows)], axis=1)
    t0 = time.perf_counter()
    oracle.attention_rows(q, k, v, 1, F, H, W, d, o1, rows, p.Bq, p.Bk, rp, ci)
    t_rows = time.perf_counter() - t0
    t_layer = G * (t_head + t_rows * N / nrows)
    dense = 4.0 * N * N * d * G
    return {
        "value": dense / t_layer / 1e12,
        "unit": "TFLOPS",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "os_cpu_count": os.cpu_count(),
        "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
        "sample": (f"head 0 of {G}: reorder Q/K/V + mask build ({t_head:.2f} s) and fp64 masked "
                   f"attention on {nrows} of {N} rows ({t_rows:.2f} s); layer time extrapolated "
                   f"as {G} x (head + rows*N/{nrows}) = {t_layer:.0f} s"),
    }


def long_clip(args, timed_steps):
    """The long-clip layer, F=33, H=45, W=80 (118,800 tokens), 24 heads, d=128,
    128x128 blocks: per step the mask is rebuilt from the current Q and K
    (COSINE of block sums, top-k at 15 % plus diagonal and temporal window),
    then bf16 attention; reorder and the fused inverse reorder as in the main
    chain."""
    import numpy as np
    import torch

    import block_sparse_attention_inverse_amd as bsa
    from block_sparse_attention_inverse_amd import synth

    cfg = synth.config(5)
    F, H, W, G, d, N = cfg["F"], cfg["H"], cfg["W"], cfg["G"], cfg["d"], cfg["N"]
    seed = synth.seed_of(5)
    orders = synth.make_orders(cfg, seed)
    log(f"[bench] long clip: generating N={N} G={G} d={d}")
    Q, K, V = synth.cast_inputs(cfg, *synth.make_qkv(cfg, orders, seed, device="cuda"))
    od = torch.from_numpy(orders).cuda()
    p = bsa.mask_params(cfg["Bq"], cfg["Bk"], 1, cfg["rho"], True, cfg["win_T"], cfg["win_r0"])
    plan = bsa.LayerPlan(G, F, H, W, d, "cuda", p, fused=True)

    def step(ev=None):
        plan.reorder_fused(Q, K, V, od)
        if ev:
            ev[0].record()
        plan.build_mask_from_sums(od)
        if ev:
            ev[1].record()
        # attention with the inverse reorder in its epilogue: O lands in
        # natural token order
        bsa.forward_natural(plan.Qp, plan.Kp, plan.Vp, plan.row_ptr, plan.col_idx, p.Bq, p.Bk,
                            od, F, H, W, out=plan.O, lse=plan.lse)
        if ev:
            ev[2].record()

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    steps = max(3, timed_steps // 2)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        evs[k][0].record()
        step(evs[k][1:])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    seg = np.array([[evs[k][i].elapsed_time(evs[k][i + 1]) for i in range(3)] for k in range(steps)])
    seg = seg.mean(axis=0)
    rp = plan.row_ptr.cpu().numpy()
    nnz = int(plan.nnz.item())
    ci = plan.col_idx[:nnz].cpu().numpy()
    nq, nk = -(-N // p.Bq), -(-N // p.Bk)
    fl = kept_flops(rp, ci, G, N, p.Bq, p.Bk, d)
    dense = 4.0 * N * N * d * G
    # the same rebuild with Top-P in place of Top-K: block scores from the
    # fused sums, then the per-row sorted Top-P cut (80 % of the softmax of
    # the COSINE scores at inverse temperature 16, log2 units; about the
    # Top-K density here) + forced blocks
    nq, nk = -(-N // p.Bq), -(-N // p.Bk)
    sc = torch.empty((G, nq, nk), dtype=torch.float32, device="cuda")
    ws_sc = torch.empty(bsa.mask_workspace(G, F, H, W, d, p), dtype=torch.uint8, device="cuda")
    ws_sel = torch.empty(bsa.scores_select_workspace(G, F, H, W, p.Bq, p.Bk), dtype=torch.uint8,
                         device="cuda")

    def topp_mask():
        bsa.block_scores(plan.sums_q, plan.sums_k, F, H, W, p, out=sc, workspace=ws_sc)
        return bsa.mask_from_scores(sc, od, F, H, W, p, top_p=0.8, temp=16.0, workspace=ws_sel)

    topp_mask()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        _, _, tnnz = topp_mask()
    e1.record()
    torch.cuda.synchronize()
    t_topp = e0.elapsed_time(e1) / steps
    topp_density = int(tnnz.item()) / (G * nq * nk)
    log(f"[bench] long clip: {wall * 1e3:.3f} ms/step; segments (ms) {seg}; top-p mask {t_topp:.3f} ms")
    return {
        "workload": "long clip: F=33,H=45,W=80 (118800 tokens), 24 heads, d=128, 128x128 blocks, "
                    "COSINE top-k 15% + diagonal + temporal window (T=2, r0=4), mask rebuilt per step",
        "steps": steps,
        "ms_per_step": wall * 1e3,
        "dense_equiv_tflops": dense / wall / 1e12,
        "block_density": nnz / (G * nq * nk),
        "kept_tflop": fl / 1e12,
        "breakdown_ms": {
            "reorder_qkv_with_qk_block_sums": float(seg[0]),
            "build_mask_from_sums": float(seg[1]),
            "attention": float(seg[2]),
            "gaps": float(wall * 1e3 - seg.sum()),
        },
        "attention_kept_tflops": fl / (seg[2] / 1e3) / 1e12,
        "attention_frac_bf16_peak": fl / (seg[2] / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "topp_mask_ms": t_topp,
        "topp_mask_density": topp_density,
        "topp_mask_policy": "top_p 0.8 of softmax(COSINE score * 16, base 2) + diagonal + window",
    }


def calibration(args):
    """Offline order calibration on the 480p-shaped layer (F=21, H=30, W=52,
    32,760 tokens, 12 heads, d=128, 64x64 blocks): for each of the six axis
    orders reorder Q and K, take the dense post-softmax map's block
    statistics (two MFMA passes over every score) and the order metric, then
    pick the argmin; then the static mask from the chosen order's block sums
    (90 % of each row's mass plus the diagonal)."""
    import numpy as np
    import torch

    import block_sparse_attention_inverse_amd as bsa
    from block_sparse_attention_inverse_amd import synth

    cfg = synth.config(3)
    F, H, W, G, d, N = cfg["F"], cfg["H"], cfg["W"], cfg["G"], cfg["d"], cfg["N"]
    B = 64
    seed = synth.seed_of(3)
    orders = synth.make_orders(cfg, seed)
    log(f"[bench] calibration: generating N={N} G={G} d={d}")
    Q, K, _ = synth.cast_inputs(cfg, *synth.make_qkv(cfg, orders, seed, device="cuda"))
    nb = (N + B - 1) // B
    stats = torch.empty((G, 6, 3), dtype=torch.float32, device="cuda")
    cnt = torch.empty((G, nb, nb), dtype=torch.int32, device="cuda")
    bsum = torch.empty((G, nb, nb), dtype=torch.float32, device="cuda")
    bmax = torch.empty((G, nb, nb), dtype=torch.float32, device="cuda")
    Qp = torch.empty((G, N, d), dtype=torch.bfloat16, device="cuda")
    Kp = torch.empty_like(Qp)
    ods = [torch.full((G,), o, dtype=torch.uint8, device="cuda") for o in range(6)]

    def step(ev=None):
        for o in range(6):
            bsa.permute(Q, ods[o], F, H, W, out=Qp)
            bsa.permute(K, ods[o], F, H, W, out=Kp)
            if ev:
                ev[2 * o].record()
            bsa.attn_block_stats(Qp, Kp, B, 1e-3, out=(cnt, bsum, bmax))
            if ev:
                ev[2 * o + 1].record()
            bsa.paro_metric(cnt, bsum, bmax, N, B, o, (9, 10), 0.02, stats)
        return bsa.paro_select(stats)

    for _ in range(max(1, args.warmup)):
        chosen = step()
    torch.cuda.synchronize()
    steps = max(2, args.steps // 10)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(12)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        chosen = step(evs[k])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    t_stats = np.mean([[evs[k][2 * o].elapsed_time(evs[k][2 * o + 1]) for o in range(6)]
                       for k in range(steps)]) / 1e3
    # the static mask from the chosen orders' block sums
    Qp2 = bsa.permute(Q, chosen, F, H, W)
    Kp2 = bsa.permute(K, chosen, F, H, W)
    _, keys, _ = bsa.attn_block_stats(Qp2, Kp2, B, 1e-3)
    bsa.mask_from_block_sums(keys, N, B, B, 0.9)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        rp, ci, nnz = bsa.mask_from_block_sums(keys, N, B, B, 0.9)
    e1.record()
    torch.cuda.synchronize()
    t_mask = e0.elapsed_time(e1) / steps
    fl = 4.0 * N * N * d * G  # two passes of S = Q.K^T over every (query, key)
    log(f"[bench] calibration: {wall * 1e3:.2f} ms for six orders; block stats {t_stats * 1e3:.3f} ms "
        f"({fl / t_stats / 1e12:.1f} TFLOP/s); static mask {t_mask:.3f} ms")
    return {
        "workload": "480p layer: F=21,H=30,W=52 (32760 tokens), 12 heads, d=128, 64x64 blocks; "
                    "six axis orders, eps=1e-3, sigma=90%, alpha=0.02; static mask at 90% row mass",
        "ms_six_orders": wall * 1e3,
        "block_stats_ms": t_stats * 1e3,
        "block_stats_tflops": fl / t_stats / 1e12,
        "block_stats_frac_bf16_peak": fl / t_stats / 1e12 / PEAK_BF16_TFLOPS,
        "static_mask_ms": t_mask,
        "static_mask_density": nnz / (G * nb * nb),
        "chosen_orders": chosen.cpu().tolist(),
        # the synthetic inputs carry a local component along each head's
        # planted axis order: how often the calibration finds it
        "planted_orders": [int(o) for o in orders],
        "heads_matching_planted": int(sum(int(a) == int(b) for a, b in zip(chosen.cpu().tolist(), orders))),
    }


HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def event_ms(fn, reps):
    """Mean duration (ms) of fn() over reps launches, HIP events on the
    current stream around the whole loop."""
    import torch

    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def graph_replay(step, eager_s, reps):
    """The whole step captured once into a HIP graph (torch.cuda.graph on a
    side stream after one eager pass there) and replayed back to back: time
    per replay beside the eager step time."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    t = event_ms(g.replay, reps)
    return {"replay_ms_per_step": t, "eager_ms_per_step": eager_s * 1e3}


def reorder_bandwidth(plan, Q, od, F, H, W, reps):
    """The reorder judged by achieved GB/s: algorithmic bytes = read + write
    of one bf16 tensor (2*N*G*d*2; indices are computed, not read), against
    the HBM peak and against a plain device copy of the same size timed in
    the same run.  The fused pass (reorder + fp32 block sums) adds its sums
    to the written bytes.  The INT8 quantiser is judged the same way: read
    bf16, write int8 codes and fp32 scales, standalone on the reordered
    tensor and fused into the reorder (codes, scales and block sums from the
    natural tensor, no bf16 copy)."""
    import torch

    import block_sparse_attention_inverse_amd as bsa

    G, N, d = plan.G, plan.N, plan.d
    nbytes = N * G * d * 2
    p = plan.params
    src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    t_copy = event_ms(lambda: dst.copy_(src), reps)
    del src, dst
    t_gather = event_ms(lambda: bsa.permute(Q, od, F, H, W, 0, out=plan.Qp), reps)
    t_scatter = event_ms(lambda: bsa.permute(plan.Qp, od, F, H, W, 1, out=plan.O), reps)
    t_fused = event_ms(lambda: bsa.permute_pool(Q, od, F, H, W, p.Bq, out=plan.Qp, sums=plan.sums_q),
                       reps)
    sums_bytes = G * -(-N // p.Bq) * d * 4
    nb = -(-N // p.Bq)
    codes = torch.empty((G, N, d), dtype=torch.int8, device="cuda")
    scales = torch.empty((G, nb), dtype=torch.float32, device="cuda")
    t_quant = event_ms(lambda: bsa.quantize_int8(plan.Qp, p.Bq, out=(codes, scales)), reps)
    t_fused8 = event_ms(lambda: bsa.permute_pool(Q, od, F, H, W, p.Bq, sums=plan.sums_q,
                                                 int8=(codes, scales), reordered=False), reps)
    del codes, scales
    quant_bytes = nbytes + nbytes // 2 + G * nb * 4  # bf16 read, int8 written, scales

    def gbs(byt, ms):
        return byt / (ms / 1e3) / 1e9

    out = {
        "tensor": f"one bf16 tensor [N][G][d] = {nbytes} bytes",
        "algorithmic_bytes": 2 * nbytes,
        "device_copy_ms": t_copy,
        "device_copy_gbs": gbs(2 * nbytes, t_copy),
        "gather_ms": t_gather,
        "gather_gbs": gbs(2 * nbytes, t_gather),
        "scatter_ms": t_scatter,
        "scatter_gbs": gbs(2 * nbytes, t_scatter),
        "fused_gather_with_block_sums_ms": t_fused,
        "fused_gather_with_block_sums_gbs": gbs(2 * nbytes + sums_bytes, t_fused),
        "quantize_int8_ms": t_quant,
        "quantize_int8_gbs": gbs(quant_bytes, t_quant),
        "fused_quantize_with_block_sums_ms": t_fused8,
        "fused_quantize_with_block_sums_gbs": gbs(quant_bytes + sums_bytes, t_fused8),
        "peak_gbs": HBM_PEAK_GBS,
    }
    out["gather_frac_peak"] = out["gather_gbs"] / HBM_PEAK_GBS
    out["gather_vs_copy"] = out["gather_gbs"] / out["device_copy_gbs"]
    out["fused_frac_peak"] = out["fused_gather_with_block_sums_gbs"] / HBM_PEAK_GBS
    out["copy_frac_peak"] = out["device_copy_gbs"] / HBM_PEAK_GBS
    out["quantize_frac_peak"] = out["quantize_int8_gbs"] / HBM_PEAK_GBS
    return out


def density_sweep(plan, plan8, Q, K, V, od, F, H, W, reps, rhos=((30, 100), (20, 100))):
    """bf16 and INT8 attention (natural-order output) at several densities on
    the same reordered inputs, with the relative L2 difference between the
    INT8 and the bf16 outputs (whole tensor, fp32)."""
    import numpy as np
    import torch

    import block_sparse_attention_inverse_amd as bsa

    G, N, d = plan.G, plan.N, plan.d
    p0 = plan.params
    plan.reorder_fused(Q, K, V, od)
    if plan8 is not None:
        plan8.reorder_fused(Q, K, V, od)
    res = {}
    for rn, rd in rhos:
        p = bsa.mask_params(p0.Bq, p0.Bk, 0, (rn, rd), True)
        rp, ci, nnz = bsa.build_mask_pooled(plan.sums_q, plan.sums_k, od, F, H, W, p)
        n = int(nnz.item())
        fl = kept_flops(rp.cpu().numpy(), ci[:n].cpu().numpy(), G, N, p.Bq, p.Bk, d)
        nq, nk = -(-N // p.Bq), -(-N // p.Bk)
        Ob = torch.empty((N, G, d), dtype=torch.bfloat16, device="cuda")
        t_b = event_ms(lambda: bsa.forward_natural(plan.Qp, plan.Kp, plan.Vp, rp, ci, p.Bq, p.Bk,
                                                   od, F, H, W, out=Ob, want_lse=False), reps)
        r = {
            "block_density": n / (G * nq * nk),
            "kept_tflop": fl / 1e12,
            "bf16_attention_ms": t_b,
            "bf16_kept_tflops": fl / (t_b / 1e3) / 1e12,
            "bf16_frac_peak": fl / (t_b / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        }
        if plan8 is not None:
            O8 = torch.empty_like(Ob)
            t_8 = event_ms(lambda: bsa.forward_int8_natural(
                plan8.Qq, plan8.sQ, plan8.Kq, plan8.sK, plan8.Vq, plan8.sV, rp, ci, p.Bq, p.Bk, od,
                F, H, W, out=O8, want_lse=False), reps)
            diff = 0.0
            ref = 0.0
            for g in range(G):  # per head in fp32, to bound the temporary memory
                a = O8[:, g].float()
                b = Ob[:, g].float()
                diff += float(torch.sum((a - b) ** 2))
                ref += float(torch.sum(b * b))
            r.update({
                "int8_attention_ms": t_8,
                "int8_kept_tops": fl / (t_8 / 1e3) / 1e12,
                "int8_frac_int8_peak": fl / (t_8 / 1e3) / 1e12 / PEAK_INT8_TOPS,
                "int8_vs_bf16_rel_l2": float(np.sqrt(diff / max(ref, 1e-30))),
            })
        res[f"rho_{rn}"] = r
        log(f"[bench] density {rn}/{rd}: {r}")
    return res


def compensation(plan, od, F, H, W, reps, Qn, Kn, Vn):
    """First-order compensation of the skipped keys on the 720p layer, after
    the bf16 forward with its natural-order output (the mask and the
    reordered tensors of the last bf16 step): its time beside the attention's,
    and its dominant product (the skip-mask GEMM over per-kv-block moments,
    2 * Nq * Nkv * (d^2 + 2d + 1) flops per head) against the bf16 peak."""
    import torch

    import block_sparse_attention_inverse_amd as bsa

    G, N, d, p = plan.G, plan.N, plan.d, plan.params
    ws = torch.empty(bsa.fo_workspace(G, N, d, p.Bq, p.Bk), dtype=torch.uint8, device="cuda")
    O = torch.empty((N, G, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((G, N), dtype=torch.float32, device="cuda")

    def fwd():
        bsa.forward_natural(plan.Qp, plan.Kp, plan.Vp, plan.row_ptr, plan.col_idx, p.Bq, p.Bk, od,
                            F, H, W, out=O, lse=lse)

    def comp():
        bsa.fo_compensate(plan.Qp, plan.Kp, plan.Vp, plan.row_ptr, plan.col_idx, p.Bq, p.Bk, O, lse,
                          od, F, H, W, workspace=ws)

    fwd()
    t_comp = event_ms(comp, reps)
    nq, nk = -(-N // p.Bq), -(-N // p.Bk)
    fl = 2.0 * nq * nk * (d * d + 2 * d + 1) * G
    # what the compensation buys: on sampled rows of a few heads, the relative
    # L2 distance of the block-sparse output to dense softmax attention (fp32
    # on the GPU, from the same bf16 inputs) without and with it
    fwd()
    O_masked = O.clone()
    comp()
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(7)
    rows = torch.randint(0, N, (1024,), generator=gen).cuda()
    sm = 1.0 / float(d) ** 0.5
    num_m = num_c = den = 0.0
    heads = [0, G // 3, (2 * G) // 3, G - 1]
    for g in heads:
        kg = Kn[:, g, :].float().contiguous()
        vg = Vn[:, g, :].float().contiguous()
        qs = Qn[rows, g, :].float().contiguous()
        s = torch.mm(qs, kg.t().contiguous()) * sm
        ref = torch.mm(torch.softmax(s, dim=1), vg)
        num_m += float(torch.sum((O_masked[rows, g, :].float() - ref) ** 2))
        num_c += float(torch.sum((O[rows, g, :].float() - ref) ** 2))
        den += float(torch.sum(ref ** 2))
        del s
    return {
        "ms": t_comp,
        "workspace_gib": ws.numel() / 2**30,
        "skip_gemm_tflop": fl / 1e12,
        "skip_gemm_tflops_if_whole_time": fl / (t_comp / 1e3) / 1e12,
        "policy": "one expansion point per q-block row (the mean of its skipped keys), "
                  "first-order Taylor term of exp(s q.k) summed over the skipped set",
        "vs_dense_rel_l2": {
            "rows": f"1024 random tokens of heads {heads}, dense softmax attention in fp32 on the GPU",
            "block_sparse": (num_m / den) ** 0.5,
            "block_sparse_compensated": (num_c / den) ** 0.5,
        },
    }


def smi_sample():
    """One reading of the GPU's socket power (W) and its per-XCD graphics
    clocks (MHz) from amd-smi, or None where the tool is not there."""
    import re
    import subprocess

    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "-g", "0"], capture_output=True,
                           text=True, timeout=30)
    except (OSError, subprocess.SubprocessError):
        return None
    pw = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", r.stdout)
    clk = [float(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", r.stdout)]
    if pw is None or not clk:
        return None
    return float(pw.group(1)), clk


def power_probe(fns, seconds):
    """Socket power and graphics clocks while each workload runs back to back
    for about `seconds` (amd-smi sampled from a second thread, readings in the
    first and last half second dropped), beside the workload's own time per
    launch.  The first sample is taken idle, 3 s after the preceding work."""
    import math
    import threading

    import torch

    torch.cuda.synchronize()
    time.sleep(3.0)  # let the averaged power reading settle after the preceding legs
    idle = smi_sample()
    if idle is None:
        return None
    out = {"idle_socket_w": idle[0], "idle_gfx_mhz_mean": sum(idle[1]) / len(idle[1]),
           "tool": "amd-smi metric -p -c (SOCKET_POWER, GFX_n CLK)"}
    for name, fn, est_ms, flop, peak in fns:
        n = max(3, math.ceil(seconds * 1e3 / est_ms))
        fn()
        torch.cuda.synchronize()
        samples, stop = [], threading.Event()

        def sampler():
            while not stop.is_set():
                t = time.perf_counter()
                r = smi_sample()
                if r is not None:
                    samples.append((t, r))
                stop.wait(0.25)

        th = threading.Thread(target=sampler)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        th.start()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        stop.set()
        th.join()
        ms = e0.elapsed_time(e1) / n
        keep = [r for t, r in samples if t0 + 0.5 <= t <= t1 - 0.5]
        rec = {"launches": n, "ms_per_launch": ms, "tflops": flop / (ms / 1e3) / 1e12, "samples": len(keep)}
        if keep:
            rec["socket_w_mean"] = sum(r[0] for r in keep) / len(keep)
            clks = [c for r in keep for c in r[1]]
            rec["gfx_mhz_mean"] = sum(clks) / len(clks)
            rec["gfx_mhz_min"] = min(clks)
            rec["gfx_mhz_max"] = max(clks)
            if peak is not None:
                # the nominal peak holds at 2.4 GHz; scaled to the clock measured under this load
                rec["frac_of_peak_at_measured_clock"] = rec["tflops"] / (peak * rec["gfx_mhz_mean"] / 2400.0)
        out[name] = rec
        log(f"[bench] power {name}: {rec}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-int8", action="store_true")
    ap.add_argument("--no-calib", action="store_true",
                    help="skip the offline order calibration timing")
    ap.add_argument("--no-long-clip", action="store_true",
                    help="skip the long-clip layer (dynamic COSINE mask rebuilt every step)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the reorder bandwidth and the 30 %% / 20 %% density sweep")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the power and clock readings (amd-smi) under the attention kernels "
                         "and a vendor bf16 GEMM")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run 3 plain device copies of 2 GiB (reference dispatches for "
                         "the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); "
              "the path shards by head across GPUs and is not run multi-GPU here.", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_attention_inverse_amd as bsa
    from block_sparse_attention_inverse_amd import synth

    cfg = synth.config(4)
    F, H, W, G, d, N = cfg["F"], cfg["H"], cfg["W"], cfg["G"], cfg["d"], cfg["N"]
    seed = synth.seed_of(4)
    orders = synth.make_orders(cfg, seed)
    log(f"[bench] generating 720p inputs N={N} G={G} d={d}")
    Q, K, V = synth.cast_inputs(cfg, *synth.make_qkv(cfg, orders, seed, device="cuda"))
    od = torch.from_numpy(orders).cuda()
    p = bsa.mask_params(cfg["Bq"], cfg["Bk"], 0, cfg["rho"], True)
    plan = bsa.LayerPlan(G, F, H, W, d, "cuda", p, fused=True)
    plan8 = None if args.no_int8 else bsa.LayerPlan(G, F, H, W, d, "cuda", p, int8=True, fused=True)
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 copies of {COPY_BYTES} bytes")
        del src, dst

    def step_bf16(ev=None):
        # reorder with the block sums of Q and K in the same pass
        plan.reorder_fused(Q, K, V, od)
        if ev:
            ev[0].record()
        plan.build_mask_from_sums(od)
        if ev:
            ev[1].record()
        # attention with the inverse reorder in its epilogue: O lands in
        # natural token order
        bsa.forward_natural(plan.Qp, plan.Kp, plan.Vp, plan.row_ptr, plan.col_idx, p.Bq, p.Bk,
                            od, F, H, W, out=plan.O, lse=plan.lse)
        if ev:
            ev[2].record()

    def step_bf16_unfused(ev=None):
        bsa.permute(Q, od, F, H, W, 0, out=plan.Qp)
        bsa.permute(K, od, F, H, W, 0, out=plan.Kp)
        bsa.permute(V, od, F, H, W, 0, out=plan.Vp)
        if ev:
            ev[0].record()
        plan.build_mask(od)
        if ev:
            ev[1].record()
        bsa.forward(plan.Qp, plan.Kp, plan.Vp, plan.row_ptr, plan.col_idx, p.Bq, p.Bk,
                    out=plan.Op, lse=plan.lse)
        if ev:
            ev[2].record()
        bsa.permute(plan.Op, od, F, H, W, 1, out=plan.O)

    def step_int8(ev=None):
        # one pass per tensor: INT8 codes and scales (+ Q/K block sums)
        plan8.reorder_fused(Q, K, V, od)
        plan8.build_mask_from_sums(od)
        if ev:
            ev[0].record()
        bsa.forward_int8_natural(plan8.Qq, plan8.sQ, plan8.Kq, plan8.sK, plan8.Vq, plan8.sV,
                                 plan8.row_ptr, plan8.col_idx, p.Bq, p.Bk, od, F, H, W,
                                 out=plan8.O, lse=plan8.lse)
        if ev:
            ev[1].record()

    sics_ws = torch.empty(bsa.order_workspace(G, F, H, W, min(p.Bq, p.Bk)), dtype=torch.uint8,
                          device="cuda")
    sq_buf = torch.empty((G, 6), dtype=torch.float32, device="cuda")
    sk_buf = torch.empty_like(sq_buf)

    def step_sics(ev=None):
        bsa.order_scores(Q, F, H, W, p.Bq, out=sq_buf, workspace=sics_ws)
        bsa.order_scores(K, F, H, W, p.Bk, out=sk_buf, workspace=sics_ws)
        bsa.select_orders(sq_buf, sk_buf)

    seg_stats = {}

    def timed(step, nev, label):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev + 1)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            evs[s][0].record()
            step(evs[s][1:])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.steps
        seg = np.array([[evs[s][k].elapsed_time(evs[s][k + 1]) for k in range(nev)]
                        for s in range(args.steps)])
        log(f"[bench] {label}: {wall * 1e3:.3f} ms/step; segments (ms) {seg.mean(axis=0)}")
        seg_stats[label] = seg
        return wall, seg.mean(axis=0)

    log("[bench] bf16 chain")
    wall, seg = timed(step_bf16, 3, "bf16")
    log("[bench] bf16 chain, unfused reorder and pooling")
    wall_u, seg_u = timed(step_bf16_unfused, 3, "bf16 unfused")
    log("[bench] SICS order selection")
    wall_s, _ = timed(step_sics, 0, "sics")
    rp_h = plan.row_ptr.cpu().numpy()
    nnz = int(plan.nnz.item())
    ci_h = plan.col_idx[:nnz].cpu().numpy()
    nq, nk = -(-N // p.Bq), -(-N // p.Bk)
    fl_kept = kept_flops(rp_h, ci_h, G, N, p.Bq, p.Bk, d)
    dense = 4.0 * N * N * d * G
    t_fwd = seg[2] / 1e3
    achieved = fl_kept / t_fwd / 1e12
    traffic = read_traffic(fl_kept)
    result = {
        "metric": METRIC,
        "value": dense / wall / 1e12,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "720p DiT attention layer: F=21,H=45,W=80 (75600 tokens), 40 heads, d=128, "
                        "128x64 blocks, DOT top-k 30% + diagonal, bf16",
            "tokens": N, "heads": G, "head_dim": d, "block": [p.Bq, p.Bk],
            "rho": p.rho_num / p.rho_den,
            "block_density": nnz / (G * nq * nk),
            "kept_tflop": fl_kept / 1e12,
            "dense_tflop": dense / 1e12,
        },
        "roofline": {
            "kernel": "bsa_forward (fwd_bf16_kernel<128,128,64>)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
        },
        "breakdown_ms": {
            "reorder_qkv_with_qk_block_sums": float(seg[0]),
            "build_mask_from_sums": float(seg[1]),
            "attention": float(seg[2]),
            "gaps": float(wall * 1e3 - seg.sum()),
        },
        "attention_ms_median": float(np.median(seg_stats["bf16"][:, 2])),
        "attention_ms_min": float(np.min(seg_stats["bf16"][:, 2])),
        "overhead_share_of_step": {
            "reorder_qkv_with_qk_block_sums": float(seg[0]) / (wall * 1e3),
            "build_mask_from_sums": float(seg[1]) / (wall * 1e3),
        },
        "unfused_ms": {
            "step": wall_u * 1e3,
            "reorder_qkv": float(seg_u[0]),
            "build_mask_with_pooling": float(seg_u[1]),
        },
        "order_selection_ms": wall_s * 1e3,
        "kept_tflops_attention": achieved,
        "dense_equiv_tflops_attention": dense / t_fwd / 1e12,
    }
    if not args.no_int8:
        log("[bench] int8 chain")
        wall8, seg8 = timed(step_int8, 2, "int8")
        t8 = seg8[1] / 1e3
        result["int8"] = {
            "ms_per_step": wall8 * 1e3,
            "dense_equiv_tflops": dense / wall8 / 1e12,
            "attention_ms": float(seg8[1]),
            "attention_kept_tops": fl_kept / t8 / 1e12,
            "frac_int8_peak": fl_kept / t8 / 1e12 / PEAK_INT8_TOPS,
            "frac_bf16_peak": fl_kept / t8 / 1e12 / PEAK_BF16_TFLOPS,
        }
    if not args.no_extras:
        log("[bench] reorder bandwidth")
        result["permute"] = reorder_bandwidth(plan, Q, od, F, H, W, reps=max(5, args.steps // 2))
        log("[bench] density sweep (30 % and 20 %)")
        result["density"] = density_sweep(plan, plan8, Q, K, V, od, F, H, W,
                                          reps=max(3, args.steps // 4))
        log("[bench] the step captured into a HIP graph")
        result["graph"] = graph_replay(step_bf16, wall, reps=max(5, args.steps // 2))
        log(f"[bench] graph: {result['graph']}")
        log("[bench] first-order compensation")
        step_bf16()
        result["compensation"] = compensation(plan, od, F, H, W, reps=max(3, args.steps // 4),
                                              Qn=Q, Kn=K, Vn=V)
        log(f"[bench] compensation: {result['compensation']}")
    if not args.no_power:
        log("[bench] power and clocks")
        gm = 8192
        ga = torch.randn(gm, gm, device="cuda", dtype=torch.bfloat16)
        gb = torch.randn(gm, gm, device="cuda", dtype=torch.bfloat16)
        gc = torch.empty(gm, gm, device="cuda", dtype=torch.bfloat16)
        fns = [("bf16_attention", lambda: bsa.forward_natural(
                    plan.Qp, plan.Kp, plan.Vp, plan.row_ptr, plan.col_idx, p.Bq, p.Bk, od, F, H, W,
                    out=plan.O, lse=plan.lse), seg[2], fl_kept, PEAK_BF16_TFLOPS)]
        if not args.no_int8:
            fns.append(("int8_attention", lambda: bsa.forward_int8_natural(
                plan8.Qq, plan8.sQ, plan8.Kq, plan8.sK, plan8.Vq, plan8.sV, plan8.row_ptr,
                plan8.col_idx, p.Bq, p.Bk, od, F, H, W, out=plan8.O, lse=plan8.lse),
                result["int8"]["attention_ms"], fl_kept, PEAK_INT8_TOPS))
        fns.append(("torch_mm_bf16_8192", lambda: torch.mm(ga, gb, out=gc), 0.8, 2.0 * gm ** 3,
                    PEAK_BF16_TFLOPS))
        step_bf16()
        result["power"] = power_probe(fns, seconds=4.0)
        del ga, gb, gc
    if not args.no_long_clip:
        result["long_clip"] = long_clip(args, timed_steps=args.steps)
    if not args.no_calib:
        result["calibration"] = calibration(args)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(cfg, Q, K, V, orders, p)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
