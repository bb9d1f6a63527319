"""Benchmark of one layer-step of PackForcing's per-block context attention on
one MI355X.

A step is the whole path on the default single-layer workload (6,240 queries,
12 heads, 27,872 keys = 12,480 sink + 16 x 182 selected from a 40-block pool
+ 6,240 recent + 6,240 current):
  pf_score_select -> pf_selection_deltas -> pf_rope_shift -> pf_partition_attn
Each step moves the recent block one block forward in time (as the next
generated block does), so every selected block gets a non-zero shift.

Prints one JSON line. `value` is partition-attention TFLOP/s over the whole
step (4 n_q n_k 128 H flops per step / step time); the per-kernel times,
the attention kernel's roofline and the CPU oracle's rate are alongside.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU (the 2.5 PFLOP/s figure)
PEAK_HBM_GBS = 8000.0
SETTLE_STEPS = 15          # untimed layer-steps before any timing, whatever --warmup says
PMC_FILE = os.path.join(ROOT, "profiles", "partition_attn_default_hbm_counters.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the batched selection/RoPE measurement (profiling the layer-step alone)")
    ap.add_argument("--batched-only", action="store_true",
                    help="only run the batched selection/RoPE measurement (for its own profile)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-c4", action="store_true", help="skip the unbounded 748,800-key contrast")
    ap.add_argument("--layer-step-only", action="store_true",
                    help="only the warm-up and timed layer-steps (for profiling their kernels)")
    ap.add_argument("--c4-only", action="store_true",
                    help="time only the unbounded 748,800-key attention (for profiling it)")
    ap.add_argument("--hr-only", action="store_true",
                    help="time only the HR-branch compressor (for profiling its kernels)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for HBM counter calibration)")
    return ap.parse_args()


def attn_flops(n_q, n_k, heads):
    return 4.0 * n_q * n_k * 128 * heads


def stats(ms):
    """Mean, median and the 10th / 90th percentiles of per-launch times (ms)."""
    ms = np.asarray(ms, dtype=np.float64)
    return {"n": int(ms.size), "mean": round(float(ms.mean()), 5), "median": round(float(np.median(ms)), 5),
            "p10": round(float(np.percentile(ms, 10)), 5), "p90": round(float(np.percentile(ms, 90)), 5)}


def kernel_source_sha(text=None):
    """Hash of the attention kernel's source with comments and blank space
    removed, so that only a change to the code voids the stored counters."""
    if text is None:
        with open(os.path.join(ROOT, "bounded_kv_cache_pf_amd", "csrc", "pf_attn.hip")) as f:
            text = f.read()
    code = [re.sub(r"//.*$", "", line).strip() for line in text.splitlines()]
    return hashlib.sha256("\n".join(c for c in code if c).encode()).hexdigest()[:16]


def counters_for_current_source():
    """The committed counter summary of the attention kernel, if it was taken
    on the current kernel source (else None)."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    return d if d.get("source_sha") == kernel_source_sha() else None


def traffic_from_counters():
    """HBM bytes per attention launch from the committed counter summary."""
    d = counters_for_current_source()
    return None if d is None else d.get("hbm_bytes_per_launch")


def mfma_busy_from_counters():
    """The attention kernel's MFMA busy fraction (busy cycles over all SIMD
    cycles of the dispatch, at the clock it ran at) from the committed counters."""
    d = counters_for_current_source()
    m = None if d is None else d.get("mfma")
    return None if m is None else round(m["mfma_busy_frac"], 4)


def host_info():
    """CPU model, usable cores and numpy's BLAS, for the CPU figures."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
                       if i.get("user_api") == "blas"})
    except Exception:  # noqa: BLE001 - informational only
        blas = []
    return {"cpu_model": model, "cores": len(os.sched_getaffinity(0)), "blas": ", ".join(blas) or "unknown"}


def _oracle_attention_pool(O, q, ks, vs, workers, chunk=256):
    """The oracle's attention on every (head, 256-query chunk) as its own task,
    over a thread pool, each task's BLAS on one thread."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    n_q, H = q.shape[0], q.shape[1]
    tasks = [(h, r0) for h in range(H) for r0 in range(0, n_q, chunk)]

    def run(t):
        h, r0 = t
        O.attn_partitioned(q[r0:r0 + chunk, h:h + 1], [k[:, h:h + 1] for k in ks], [v[:, h:h + 1] for v in vs])

    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(run, tasks))


def cpu_baseline(cache, cfg, seconds):
    """The oracle's layer-step on the host cores: selection, placement and the
    RoPE shift by the oracle's own functions, then its attention split into
    (head, 256-query chunk) tasks over a pool of one worker per usable core.
    Whole steps repeat for about `seconds` of wall time; if one step would take
    far longer, the attention covers only the first query rows."""
    import oracle as O
    info = host_info()
    workers = min(info["cores"], 16)    # one GPU's share of the host cores
    tags = O.initial_pos_tags(cfg.pool_blocks, cfg.sink_blocks, cfg.block_frames)
    fr = (cfg.sink_blocks + cfg.pool_blocks) * cfg.block_frames

    def step(rows):
        scores = O.block_scores(cache["q"], cache["pool_k"], cfg.n_c)
        ids = O.select_topk(scores, cfg.top_k)
        deltas, _ = O.placement_deltas(ids, tags, fr, cfg.block_frames)
        pool_k = O.rope_shift_blocks(cache["pool_k"], cfg.n_c, ids, deltas)
        ks, vs = O.partitions(dict(cache, pool_k=pool_k), cfg.n_c, ids)
        _oracle_attention_pool(O, cache["q"][:rows], ks, vs, workers)

    cal_rows = 512
    t0 = time.perf_counter()
    step(cal_rows)
    t_cal = time.perf_counter() - t0
    est_full = t_cal * cfg.n / cal_rows
    if est_full > 2 * seconds:          # one whole step is too long: sample query rows
        rows = max(256, (int(cfg.n * seconds / est_full) // 256) * 256)
        t0 = time.perf_counter()
        step(rows)
        dt = time.perf_counter() - t0
        n_steps, what = 1, f"one layer-step with attention for the first {rows} of {cfg.n} query rows"
    else:
        rows, n_steps, dt = cfg.n, 0, 0.0
        while dt < seconds:
            t0 = time.perf_counter()
            step(cfg.n)
            dt += time.perf_counter() - t0
            n_steps += 1
        what = f"{n_steps} whole layer-step(s) (all {cfg.n} query rows)"
    tflops = n_steps * attn_flops(rows, cfg.n_keys, cfg.heads) / dt / 1e12
    return {"value": round(tflops, 4), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"the fp64 numpy oracle on the bench workload: {what} -- scoring of all queries over "
                      f"the {cfg.pool_blocks}-block pool, top-{cfg.top_k} selection, placement, RoPE shift, "
                      f"then attention over all {cfg.n_keys} keys as (head, 256-query chunk) tasks on "
                      f"{workers} worker threads with one BLAS thread each; {dt:.1f} s wall; value = attention "
                      f"flops of the sample / wall time",
            "cpu_model": info["cpu_model"], "blas": info["blas"], "threads_per_worker": 1,
            "seconds": round(dt, 2), "rows": rows, "layer_steps": n_steps}


def hbm_batched(pf, torch, cfg_pool, layers, reps):
    """Selection, placement and RoPE shift batched over `layers` independent caches
    at the 116-block pool shapes (the full 30-layer generation step's per-step
    selection work). Returns achieved algorithmic GB/s of the HBM-bound calls."""
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg_pool.seed)
    H, n, n_c, M, k, Bf = cfg_pool.heads, cfg_pool.n, cfg_pool.n_c, cfg_pool.pool_blocks, cfg_pool.top_k, \
        cfg_pool.block_frames
    s = cfg_pool.scale
    q = (torch.randn((layers, n, H, 128), generator=g, device="cuda") * s).to(torch.bfloat16)
    pk = torch.randn((layers, M, n_c, H, 128), generator=g, device="cuda") * s
    pk += torch.randn((layers, M, 1, H, 128), generator=g, device="cuda") * cfg_pool.pool_offset_std
    pk = pk.to(torch.bfloat16).reshape(layers, M * n_c, H, 128)
    tags = ((cfg_pool.sink_blocks + torch.arange(M, device="cuda", dtype=torch.int32)) * Bf).repeat(layers, 1)
    tags = tags.contiguous()
    ids = torch.empty((layers, k), dtype=torch.int32, device="cuda")
    scores = torch.empty((layers, M), dtype=torch.float32, device="cuda")
    deltas = torch.empty((layers, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(pf.pf_score_select_batched_workspace_bytes(n, H, M, n_c, layers), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps + 2)]
    for i in range(reps + 2):
        fr = (cfg_pool.sink_blocks + M + i) * Bf
        ev[i][0].record(stream)
        pf.pf_score_select_batched(q, pk, n_c, k, ids_out=ids, scores_out=scores, workspace=ws)
        ev[i][1].record(stream)
        pf.pf_selection_deltas_batched(ids, tags, fr, Bf, deltas_out=deltas)
        ev[i][2].record(stream)
        pf.pf_rope_shift_batched(pk, n_c, deltas, ids)
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    t = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in ev[2:]]).mean(axis=0)
    row = H * 128 * 2
    sel_bytes = layers * row * (n + M * n_c)
    rope_bytes = layers * k * n_c * H * 2 * 88
    out = {"workload": f"{layers} independent caches at the {M}-block pool shapes ({n} queries x {H} heads, "
                       f"pool {M} x {n_c} rows, top-{k}), one batched call each",
           "score_select": {"ms": round(float(t[0]), 4), "algorithmic_bytes": sel_bytes,
                            "GB/s": round(sel_bytes / (t[0] * 1e-3) / 1e9, 1),
                            "frac_hbm": round(sel_bytes / (t[0] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
           "selection_deltas": {"ms": round(float(t[1]), 4)},
           "rope_shift": {"ms": round(float(t[2]), 4), "algorithmic_bytes": rope_bytes,
                          "GB/s": round(rope_bytes / (t[2] * 1e-3) / 1e9, 1),
                          "frac_hbm": round(rope_bytes / (t[2] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}}
    del q, pk, ws
    # the pages' eviction event: every layer's sink slab shifted forward by
    # delta = evicted blocks x B_f, one batched call over the layers
    sink = (torch.randn((layers, cfg_pool.n_sink, H, 128), generator=g, device="cuda") * s).to(torch.bfloat16)
    sd = torch.full((layers, 1), 2 * Bf, dtype=torch.int32, device="cuda")
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps + 2)]
    for i in range(reps + 2):
        sev[i][0].record(stream)
        pf.pf_rope_shift_batched(sink, cfg_pool.n_sink, sd)
        sev[i][1].record(stream)
    torch.cuda.synchronize()
    ts = float(np.mean([e[0].elapsed_time(e[1]) for e in sev[2:]]))
    sink_bytes = layers * cfg_pool.n_sink * H * 2 * 88
    out["sink_shift"] = {"workload": f"{layers} sink slabs of {cfg_pool.n_sink} rows, one batched call",
                         "ms": round(ts, 4), "algorithmic_bytes": sink_bytes,
                         "GB/s": round(sink_bytes / (ts * 1e-3) / 1e9, 1),
                         "frac_hbm": round(sink_bytes / (ts * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del sink
    # The shift reads and writes whole 128-byte lines: the first line of each
    # 256-byte row-head holds the 88 bytes of temporal dims, so 256 bytes move
    # per 176 algorithmic (a layout ceiling of 68.75% of peak). Its line rate
    # is set against a plain device copy (read + write) measured here.
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(7)]
    for e in cev:
        e[0].record(stream)
        b.copy_(a)
        e[1].record(stream)
    torch.cuda.synchronize()
    tc = float(np.median([e[0].elapsed_time(e[1]) for e in cev[2:]]))
    copy_gbs = 2 * a.numel() / (tc * 1e-3) / 1e9
    del a, b
    out["copy_reference"] = {"workload": "1 GiB device copy (torch copy_), bytes read + written",
                             "ms": round(tc, 4), "GB/s": round(copy_gbs, 1),
                             "frac_hbm": round(copy_gbs / PEAK_HBM_GBS, 4)}
    for key in ("rope_shift", "sink_shift"):
        line = out[key]["GB/s"] * 256 / 176
        out[key]["line_GB/s"] = round(line, 1)
        out[key]["line_frac_of_copy"] = round(line / copy_gbs, 4)
    return out


def selection_cadence(pf, torch, pfgen, dev, ms_attn, caches=8):
    """The pages' faster selection (a quarter of the query rows, every other
    head) against full scoring: time per call on the default layer and how many
    of the 16 selected blocks agree on caches with clear block preferences
    (per-head query mean, block-wise key offsets). The pages' two baselines are
    reported alongside: FIFO (the 16 newest blocks) and random selection
    (pf_select_random, one stream per cache)."""
    cfg = pfgen.C2Q
    k = cfg.top_k
    agree_sub, agree_fifo, agree_rand = [], [], []
    t_full, t_sub = [], []
    for i in range(caches):
        c = pfgen.make(cfg, cfg.seed + 100 + i)
        q, pk = dev(c["q"]), dev(c["pool_k"])
        full, _ = pf.pf_score_select(q, pk, cfg.n_c, k)
        sub, _ = pf.pf_score_select_sub(q, pk, cfg.n_c, k, 4, 2)
        fs, ss = set(full.cpu().numpy().tolist()), set(sub.cpu().numpy().tolist())
        agree_sub.append(len(fs & ss) / k)
        agree_fifo.append(len(fs & set(range(cfg.pool_blocks - k, cfg.pool_blocks))) / k)
        rnd = pf.pf_select_random(cfg.pool_blocks, k, 2024, i)
        agree_rand.append(len(fs & set(rnd.cpu().numpy().tolist())) / k)
        for fn, acc in ((lambda: pf.pf_score_select(q, pk, cfg.n_c, k), t_full),
                        (lambda: pf.pf_score_select_sub(q, pk, cfg.n_c, k, 4, 2), t_sub)):
            fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                fn()
            e1.record()
            torch.cuda.synchronize()
            acc.append(e0.elapsed_time(e1) / 10)
    return {"workload": f"{caches} caches at the 116-block pool shapes with a per-head query mean; "
                        f"sub-sampled = every 4th query row and every other head",
            "full_ms": round(float(np.median(t_full)), 4), "subsampled_ms": round(float(np.median(t_sub)), 4),
            "subsampled_topk_agreement": round(float(np.mean(agree_sub)), 4),
            "fifo_topk_agreement": round(float(np.mean(agree_fifo)), 4),
            "random_topk_agreement": round(float(np.mean(agree_rand)), 4),
            "random_expected_agreement": round(k / cfg.pool_blocks, 4),
            "full_over_attention": round(float(np.median(t_full)) / ms_attn, 4)}


def rollin_overlap(pf, torch, pfgen, step_attn, layers=30, reps=10):
    """The dual-resolution roll-in of every layer's new compressed block (one
    batched call) on a second stream, overlapped with a layer's attention on
    the launch stream: attention time alone, roll-in alone, and both."""
    cfg = pfgen.C2
    H, n_c = cfg.heads, cfg.n_c
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed + 7)
    blk = (torch.randn((2, layers, n_c, H, 128), generator=g, device="cuda") * cfg.scale).to(torch.bfloat16)
    pool = torch.zeros((2, layers, 2 * n_c, H, 128), dtype=torch.bfloat16, device="cuda")
    tags = torch.zeros((layers, 2), dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    roll = lambda: pf.pf_rollin_batched(pool[0], pool[1], tags, 1, blk[0], blk[1], 0, stream=side)

    def timed(fn, stream):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    attn_ms = timed(step_attn, main)
    roll_ms = timed(roll, side)

    def both():
        side.wait_stream(main)
        roll()
        step_attn()
        main.wait_stream(side)
    both_ms = timed(both, main)
    return {"workload": f"{layers} compressed {n_c}-row blocks rolled in on a second stream during one "
                        f"default layer-step attention",
            "attn_ms": round(attn_ms, 4), "rollin_ms": round(roll_ms, 4), "attn_with_rollin_ms": round(both_ms, 4)}


def hr_branch(pf, torch, pfgen, dev, gen_ms, reps=20):
    """The HR-branch compressor on the default latent block (4 frames of
    60 x 104 x 16 channels -> 182 tokens x 1536) with seeded weights: the whole
    branch at batch 1 (one block, as it runs once per generated block) and
    batch 8, and each strided stage alone at batch 1 with its own roofline
    (algorithmic flops 2 M N K; bytes = input + weights + bias + output)."""
    lat = pfgen.HR_LATENT
    T, H, W, C = lat["frames"], lat["height"], lat["width"], lat["channels"]
    stages, (wp, bp) = pfgen.hr_weights(3001)
    ds = [(dev(w), torch.from_numpy(b).cuda()) for w, b in stages]
    dp = (dev(wp), torch.from_numpy(bp).cuda())
    stream = torch.cuda.current_stream()

    def timed(fn):
        # these launches are shorter than the host cost of a call, so the reps
        # are captured once in a HIP graph and the graph's replay is timed
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {"workload": f"HR branch on {T}x{H}x{W}x{C} latent blocks, widths {list(pfgen.HR_WIDTHS)} -> "
                       f"{pfgen.HR_HIDDEN}, seeded weights"}
    rows, flops_block = [], 0
    t, h, w, c = T, H, W, C
    layers = [(wd, k, True, st) for wd, k, st in zip(pfgen.HR_WIDTHS, pfgen.HR_KERNELS, ds)]
    layers.append((pfgen.HR_HIDDEN, (1, 1, 1), False, (dp[0].view(pfgen.HR_HIDDEN, 1, 1, 1, -1), dp[1])))
    for wd, (kt, kh, kw), act, (wt, bt) in layers:
        x = torch.randn((1, t, h, w, c), device="cuda").to(torch.bfloat16)
        to, ho, wo = t // kt, h // kh, w // kw
        M, K = to * ho * wo, kt * kh * kw * c
        y = torch.empty((1, to, ho, wo, wd), dtype=torch.bfloat16, device="cuda")
        need = pf.pf_hr_conv_workspace_bytes(1, t, h, w, c, (kt, kh, kw), wd)
        wsb = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        ms = timed(lambda: pf.pf_hr_conv(x, wt, bt, (kt, kh, kw), act=act, y=y, workspace=wsb))
        fl = 2 * M * wd * K
        by = (to * kt * ho * kh * wo * kw * c + wd * K + M * wd) * 2 + wd * 4
        flops_block += fl
        intensity = fl / by
        bound = "mfma" if intensity > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"
        frac = (fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS) if bound == "mfma" else (by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS)
        rows.append({"kernel": f"{kt}x{kh}x{kw}", "c_in": c, "c_out": wd, "M": M, "K": K, "ms": round(ms, 4),
                     "flops": fl, "bytes": by, "bound": bound, "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1),
                     "GB/s": round(by / (ms * 1e-3) / 1e9, 1), "frac": round(frac, 4),
                     "split_k_workspace": need})
        t, h, w, c = to, ho, wo, wd
        del x, y, wsb
    out["stages"] = rows
    out["flops_per_block"] = flops_block
    for batch in (1, 8):
        z = torch.randn((batch, T, H, W, C), device="cuda").to(torch.bfloat16)
        o = torch.empty((batch, (T // 2) * (H // 8) * (W // 8), pfgen.HR_HIDDEN), dtype=torch.bfloat16, device="cuda")
        wsb = torch.empty(pf.pf_hr_branch_workspace_bytes(batch, T, H, W, C, pfgen.HR_WIDTHS, pfgen.HR_HIDDEN),
                          dtype=torch.uint8, device="cuda")
        ms = timed(lambda: pf.pf_hr_branch(z, ds, dp, out=o, workspace=wsb))
        out[f"batch{batch}_ms"] = round(ms, 4)
        out[f"batch{batch}_tflops"] = round(batch * flops_block / (ms * 1e-3) / 1e12, 1)
        del z, o, wsb
    # the branch runs once per generated block, whose generation takes
    # layers x denoising steps layer-steps
    out["frac_of_generation_step"] = round(out["batch1_ms"] / gen_ms, 6)
    return out


def generation_step(pf, torch, cfg, reps=2, cadence=False):
    """One full generation step at the 2-minute pool shapes: every layer keeps
    its own resident cache (sink, a 117-slot pool holding 116 blocks, recent,
    current) and for each of the denoising steps runs select-and-place, the
    RoPE shift and the attention; after the steps every layer's new compressed
    block rolls into slot 116 in one batched call. Queries are drawn once per
    layer (the kernels do not depend on their values' provenance).

    cadence=True follows the pages instead of rerunning selection every step:
    each layer selects once, at the block's first denoising step, with the
    faster sub-sampled scoring (every 4th query row, every other head), places
    and shifts; the later steps reuse the ids and the shifted keys (their
    placement would give delta 0). The selection's share of the step is
    reported against the pages' figure of under 1%."""
    L, S = cfg.layers, cfg.steps
    H, n, n_c, M, k, Bf = cfg.heads, cfg.n, cfg.n_c, cfg.pool_blocks, cfg.top_k, cfg.block_frames
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed)

    def draw(rows):
        return (torch.randn((rows, H, 128), generator=g, device="cuda") * cfg.scale).to(torch.bfloat16)

    layers = []
    for _ in range(L):
        c = {"q": draw(n), "sink_k": draw(cfg.n_sink), "sink_v": draw(cfg.n_sink),
             "pool_k": draw((M + 1) * n_c), "pool_v": draw((M + 1) * n_c), "recent_k": draw(cfg.n_recent),
             "recent_v": draw(cfg.n_recent), "cur_k": draw(n), "cur_v": draw(n),
             "tags": ((cfg.sink_blocks + torch.arange(M, device="cuda", dtype=torch.int32)) * Bf).contiguous(),
             "ids": torch.empty(k, dtype=torch.int32, device="cuda"),
             "deltas": torch.empty(k, dtype=torch.int32, device="cuda"),
             "scores": torch.empty(M, dtype=torch.float32, device="cuda")}
        layers.append(c)
    blk = torch.stack([draw(n_c) for _ in range(2 * L)]).view(2, L, n_c, H, 128)
    pool_k_all = [c["pool_k"] for c in layers]
    ws = torch.empty(max(pf.pf_score_select_workspace_bytes(n, H, M, n_c),
                         pf.pf_score_select_sub_workspace_bytes(n, H, 4, 2, M, n_c)), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((n, H, 128), dtype=torch.bfloat16, device="cuda")
    aws = torch.empty(max(pf.pf_partition_attn_workspace_bytes(n, H, cfg.n_keys), 1), dtype=torch.uint8,
                      device="cuda")
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    fr = (cfg.sink_blocks + M) * Bf

    def select(c, pk):
        if cadence:
            pf.pf_score_select_sub(c["q"], pk, n_c, k, 4, 2, ids_out=c["ids"], scores_out=c["scores"],
                                   workspace=ws)
            pf.pf_selection_deltas(c["ids"], c["tags"], fr, Bf, deltas_out=c["deltas"])
        else:
            pf.pf_select_place(c["q"], pk, n_c, k, c["tags"], fr, Bf, ids_out=c["ids"], deltas_out=c["deltas"],
                               scores_out=c["scores"], workspace=ws)

    def one_step():
        for s_i in range(S):
            for c in layers:
                pk = c["pool_k"][:M * n_c]
                pv = c["pool_v"][:M * n_c]
                if s_i == 0 or not cadence:
                    select(c, pk)
                    pf.pf_rope_shift(pk, n_c, c["deltas"], c["ids"])
                pf.pf_partition_attn(c["q"], c["sink_k"], c["sink_v"], pk, pv, n_c, c["ids"], c["recent_k"],
                                     c["recent_v"], c["cur_k"], c["cur_v"], o=o, workspace=aws)
        # every layer's new compressed block into pool slot M, on a second stream
        side.wait_stream(main)
        for li, c in enumerate(layers):
            pf.pf_rollin(c["pool_k"], c["pool_v"], None, M, blk[0, li], blk[1, li], fr, stream=side)
        main.wait_stream(side)

    one_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(main)
    for _ in range(reps):
        one_step()
    e1.record(main)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # the selection calls of one generation step alone (every layer, as often
    # as the step runs them), for their share of the step
    n_sel = L * (1 if cadence else S)
    e0.record(main)
    for i in range(n_sel):
        c = layers[i % L]
        select(c, c["pool_k"][:M * n_c])
    e1.record(main)
    torch.cuda.synchronize()
    sel_ms = e0.elapsed_time(e1)
    flops = L * S * attn_flops(n, cfg.n_keys, H)
    del layers, blk, pool_k_all
    mode = ("the pages' cadence: sub-sampled selection (every 4th query row, every other head), placement and "
            "shift at the first denoising step only" if cadence else
            "selection, placement and shift rerun at every denoising step")
    return {"workload": f"{L} layers x {S} denoising steps at the {M}-block pool shapes ({cfg.n_keys} keys per "
                        f"layer-step), then {L} roll-ins on a second stream; {mode}",
            "ms": round(ms, 3), "layer_steps": L * S, "ms_per_layer_step": round(ms / (L * S), 4),
            "attention_tflops_over_the_step": round(flops / (ms * 1e-3) / 1e12, 1),
            "selection_calls": n_sel, "selection_ms": round(sel_ms, 3),
            "selection_frac_of_step": round(sel_ms / ms, 5)}


def unbounded_c4(pf, torch, cfg, cpu=True, reps=3):
    """The pages' unbounded contrast: one layer's 6,240 queries over all 748,800
    full-resolution keys of a 2-minute video (sink + 117 recent blocks + the
    current block, no compression or selection), drawn on the device from a
    seed. Attention time and roofline; next to it the oracle's rate on a
    bounded sample (one head, 128 queries over all keys, one core), scaled
    linearly to the whole call and labelled as an extrapolation."""
    H, n = cfg.heads, cfg.n
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed)

    def draw(rows):
        return (torch.randn((rows, H, 128), generator=g, device="cuda") * cfg.scale).to(torch.bfloat16)

    q = draw(n)
    sink_k, sink_v = draw(cfg.n_sink), draw(cfg.n_sink)
    rec_k, rec_v = draw(cfg.n_recent), draw(cfg.n_recent)
    cur_k, cur_v = draw(n), draw(n)
    n_keys = cfg.n_sink + cfg.n_recent + n
    o = torch.empty_like(q)
    ws = torch.empty(max(pf.pf_partition_attn_workspace_bytes(n, H, n_keys), 1), dtype=torch.uint8, device="cuda")
    call = lambda: pf.pf_partition_attn(q, sink_k, sink_v, None, None, 1, None, rec_k, rec_v, cur_k, cur_v,
                                        o=o, workspace=ws)
    call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        call()
        e[1].record()
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    flops = attn_flops(n, n_keys, H)
    med = float(np.median(ms))
    out = {"workload": f"one layer, {n} queries x {H} heads over {n_keys} full-resolution keys "
                       f"({cfg.n_sink} sink + {cfg.n_recent} recent + {n} current), no selection",
           "flops_per_launch": flops, "ms": stats(ms),
           "tflops": round(flops / (med * 1e-3) / 1e12, 1),
           "frac_mfma_peak": round(flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "kv_bytes": int(2 * n_keys * H * 128 * 2)}
    del q, sink_k, sink_v, rec_k, rec_v, cur_k, cur_v, o, ws
    torch.cuda.empty_cache()
    if cpu:
        import oracle as O
        rng = np.random.default_rng(cfg.seed)

        def bits(rows):
            return O.f64_to_bf16(rng.standard_normal((rows, 1, 128)).astype(np.float32) * cfg.scale)
        rows = 128
        qs, ks, vs = bits(rows), bits(n_keys), bits(n_keys)
        t0 = time.perf_counter()
        O.attn_partitioned(qs, [ks], [vs])
        dt = time.perf_counter() - t0
        rate = attn_flops(rows, n_keys, 1) / dt
        out["cpu_oracle_extrapolated"] = {
            "kind": "oracle, extrapolated", "sample": f"one head, {rows} queries over all {n_keys} keys, fp64 "
                                                      f"numpy oracle, one core ({dt:.1f} s)",
            "sample_tflops": round(rate / 1e12, 5),
            "whole_call_s_one_core": round(flops / rate, 1),
            "whole_call_s_16_cores_linear": round(flops / rate / 16, 1)}
    return out


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path is single-GPU by design "
              "and runs on one MI355X.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import bounded_kv_cache_pf_amd as pf
    import pfgen

    if args.batched_only:
        print(json.dumps({"hbm_batched": hbm_batched(pf, torch, pfgen.C2, pfgen.C3.layers, args.steps)}), flush=True)
        return
    if args.c4_only:
        print(json.dumps({"unbounded_c4": unbounded_c4(pf, torch, pfgen.C4, cpu=False, reps=args.steps)}),
              flush=True)
        return
    if args.hr_only:
        def dev_bits(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
        print(json.dumps({"hr_branch": hr_branch(pf, torch, pfgen, dev_bits, gen_ms=float("nan"),
                                                 reps=args.steps)}), flush=True)
        return

    cfg = pfgen.C1
    t_gen = time.perf_counter()
    cache = pfgen.make(cfg)
    t_gen = time.perf_counter() - t_gen

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    t = {k: dev(v) for k, v in cache.items()}
    M, k, Bf = cfg.pool_blocks, cfg.top_k, cfg.block_frames
    # pool block m starts out encoding frames from (sink blocks + m) * B_f on
    tags = torch.tensor((cfg.sink_blocks + np.arange(M)) * Bf, dtype=torch.int32, device="cuda")
    ids = torch.empty(k, dtype=torch.int32, device="cuda")
    scores = torch.empty(M, dtype=torch.float32, device="cuda")
    deltas = torch.empty(k, dtype=torch.int32, device="cuda")
    ws = torch.empty(pf.pf_score_select_workspace_bytes(cfg.n, cfg.heads, M, cfg.n_c), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(t["q"])
    stream = torch.cuda.current_stream()

    aws = torch.empty(max(pf.pf_partition_attn_workspace_bytes(cfg.n, cfg.heads, cfg.n_keys), 1),
                      dtype=torch.uint8, device="cuda")

    def step(i, ev=None):
        fr = (cfg.sink_blocks + M + i) * Bf
        if ev: ev[0].record(stream)
        pf.pf_select_place(t["q"], t["pool_k"], cfg.n_c, k, tags, fr, Bf, ids_out=ids, deltas_out=deltas,
                           scores_out=scores, workspace=ws)
        if ev: ev[1].record(stream)
        pf.pf_rope_shift(t["pool_k"], cfg.n_c, deltas, ids)
        if ev: ev[2].record(stream)
        pf.pf_partition_attn(t["q"], t["sink_k"], t["sink_v"], t["pool_k"], t["pool_v"], cfg.n_c, ids,
                             t["recent_k"], t["recent_v"], t["cur_k"], t["cur_v"], o=o, workspace=aws)
        if ev: ev[3].record(stream)

    # the clock takes about a dozen attention launches to settle: the untimed
    # warm-up is topped up to SETTLE_STEPS layer-steps before anything is timed
    n_warm = max(args.warmup, SETTLE_STEPS)
    for i in range(n_warm):
        step(i)
    torch.cuda.synchronize()

    # K steps with an event after each call, for the per-call breakdown and the
    # spread of step times (these also run before the headline steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(n_warm + i, evs[i])
    torch.cuda.synchronize()
    part = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs])   # [steps, 3] ms
    ms_select, ms_rope, ms_attn = part.mean(axis=0)
    step_each = np.array([e[0].elapsed_time(e[3]) for e in evs])

    # the timed steps, with nothing between the launches
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(n_warm + args.steps + i)
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    flops = attn_flops(cfg.n, cfg.n_keys, cfg.heads)
    value = flops / (ms_step * 1e-3) / 1e12
    attn_tflops = flops / (ms_attn * 1e-3) / 1e12
    # algorithmic bytes: Q + K,V of every context key + O (bf16)
    row_bytes = cfg.heads * 128 * 2
    attn_bytes = row_bytes * (2 * cfg.n + 2 * cfg.n_keys)
    sel_bytes = row_bytes * (cfg.n + M * cfg.n_c)
    rope_bytes = 2 * k * cfg.n_c * cfg.heads * 88

    out = {
        "metric": "partition-attention TFLOP/s and ms/layer-step at 27,872 keys; % bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_layer_steps_run": n_warm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(2) bf16 caches of the pages' default shapes)",
        "config": {"workload": "default single layer-step: 6,240 queries x 12 heads x 128 over 27,872 keys "
                               "(12,480 sink + 16 of 40 compressed 182-token blocks + 6,240 recent + "
                               "6,240 current); select -> place -> RoPE shift -> attend",
                   "n_q": cfg.n, "n_keys": cfg.n_keys, "heads": cfg.heads, "pool_blocks": M, "top_k": k,
                   "n_c": cfg.n_c},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_counters(),
                     "mfma_busy_counter": mfma_busy_from_counters(),
                     "kernel": "partition_attn_kernel", "flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": attn_bytes},
        "kernels_ms": {"select_place": round(float(ms_select), 5), "rope_shift": round(float(ms_rope), 5),
                       "partition_attn": round(float(ms_attn), 5)},
        "attn_tflops": round(attn_tflops, 2),
        "attn_frac_mfma_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "select_place_gbs": round(sel_bytes / (ms_select * 1e-3) / 1e9, 1),
        "rope_shift_gbs": round(rope_bytes / (ms_rope * 1e-3) / 1e9, 1),
        "input_gen_s": round(t_gen, 2),
        "step_ms_stats": stats(step_each),
        "attn_ms_stats": stats(part[:, 2]),
        "attn_tflops_at_median": round(flops / (float(np.median(part[:, 2])) * 1e-3) / 1e12, 2),
    }
    if args.layer_step_only:
        print(json.dumps(out), flush=True)
        return
    out["selection_cadence"] = selection_cadence(pf, torch, pfgen, dev, ms_attn)
    out["rollin_overlap"] = rollin_overlap(pf, torch, pfgen, step_attn=lambda: pf.pf_partition_attn(
        t["q"], t["sink_k"], t["sink_v"], t["pool_k"], t["pool_v"], cfg.n_c, ids, t["recent_k"], t["recent_v"],
        t["cur_k"], t["cur_v"], o=o))
    out["hr_branch"] = hr_branch(pf, torch, pfgen, dev, gen_ms=pfgen.C3.layers * pfgen.C3.steps * ms_step)
    if not args.no_batched:
        out["generation_step"] = generation_step(pf, torch, pfgen.C3)
        out["generation_step_pages_cadence"] = generation_step(pf, torch, pfgen.C3, cadence=True)
    if not args.no_c4:
        out["unbounded_c4"] = unbounded_c4(pf, torch, pfgen.C4, cpu=not args.no_cpu)
    if not args.no_batched:
        hb = hbm_batched(pf, torch, pfgen.C2, pfgen.C3.layers, 5)
        # one generation step = layers x denoising steps layer-steps; the eviction
        # shift runs once per step at most
        gen_ms = pfgen.C3.layers * pfgen.C3.steps * ms_step
        hb["sink_shift"]["frac_of_generation_step"] = round(hb["sink_shift"]["ms"] / gen_ms, 5)
        out["hbm_batched"] = hb
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cache, cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
