"""Benchmark: paged-KV attention prefill on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-coverage]

One step = plan (host validation + scheduling + the task-list upload) and run
(attention + split merge) over the paged batch-prefill workload: batch 8,
qo ~ U[128, 1024], kv = qo + U[0, 2048], page 16 in a permuted pool 1.5x the
pages needed, Hq 32 / Hkv 8, head_dim 128, bf16, causal.  Inputs are resident
in HBM before the timed region.  value = algorithmic TFLOP/s over the whole
step (4 * head_dim flops per visible (query, key) pair per q head).

Inputs are cycled through device copies so that at least 512 MB of inputs is
read between two uses of one copy (the 256 MB Infinity Cache serves none of a
step's inputs).

Prints ONE JSON line.  `roofline` covers the attention kernel: its average
(and median) duration over >= 50 launches after 10 warm-ups, each launch
bracketed by HIP events on the stream it runs on.  `plan_us` is the host cost
of planning (the C-ABI call alone, and the Python binding's call).
`coverage` times every other workload of the path (windowed prefill,
non-causal windows at page 1024 and 16, speculative verify at every batch and
kv-head count, long-context split-KV with merge) against its roofline.
`cpu_baseline` times the float64 CPU oracle on a bounded sample of the same
workload (rank 0, N = 1 only).  `copy_ceiling` is the attainable HBM rate of
a plain device-to-device copy of 1 GiB (read + write bytes over its time).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "masked-attention TFLOP/s (prefill) + KV HBM GB/s (verify), fraction of peak"
# the files that define the prefill attention kernel; their joint hash tags the
# committed HBM counters
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_prefill_amd", "csrc", f)
                  for f in ("pkv_attn.h", "pkv_device.h", "pkv_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_prefill_paged_b8_hbm.txt")
VERIFY_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_verify_b64_hkv8_hbm.txt")


def kernel_source_sha():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch of an attention kernel, from a committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (already scaled by the copy-kernel
    calibration), or None when absent or taken on a different kernel source."""
    try:
        rec = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    rec[k.strip()] = v.strip()
        if rec.get("kernel_source_sha256") != kernel_source_sha():
            return None
        if "traffic_bytes_per_launch" in rec:
            return float(rec["traffic_bytes_per_launch"])
        return float(rec["fetch_bytes_per_launch"]) + float(rec["write_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def visible_pairs(w):
    """Number of (row, key) pairs the mask keeps, per q head, summed over requests."""
    total = 0
    for b in range(w.batch_size):
        Q, L = int(w.qo_lens[b]), int(w.kv_lens[b])
        if w.custom_mask is not None:   # topology bits, within the left window
            seg = w.custom_mask[int(w.mask_indptr[b]):int(w.mask_indptr[b + 1])]
            bits = np.unpackbits(seg, bitorder="little")[:Q * L].reshape(Q, L).astype(bool)
            if w.window_left >= 0:
                i = np.arange(Q)[:, None]
                j = np.arange(L)[None, :]
                bits &= j + Q + w.window_left >= L + i
            total += int(bits.sum())
            continue
        i = np.arange(Q, dtype=np.int64)
        hi = i + L - Q if w.causal else np.full(Q, L - 1)
        hi = np.minimum(hi, L - 1)
        lo = np.zeros(Q, dtype=np.int64) if w.window_left < 0 else np.maximum(0, L + i - Q - w.window_left)
        total += int(np.maximum(hi - lo + 1, 0).sum())
    return total


def attention_flops(w):
    return 4.0 * w.head_dim * w.num_qo_heads * visible_pairs(w)


def kv_bytes(w, kv_elem=2):
    """K and V rows any row of a request can see, x Hkv x 2 x D x kv_elem bytes, plus q, o, lse."""
    elem = kv_elem
    keys = 0
    for b in range(w.batch_size):
        Q, L = int(w.qo_lens[b]), int(w.kv_lens[b])
        hi = L - 1
        lo = 0 if w.window_left < 0 else max(0, L - Q - w.window_left)
        keys += hi - lo + 1
    kv = keys * w.num_kv_heads * 2 * w.head_dim * elem
    qo = 2 * w.total_q * w.num_qo_heads * w.head_dim * 2 + w.total_q * w.num_qo_heads * 4
    return kv + qo


def _device_inputs(w, dev):
    import torch
    view = torch.bfloat16 if w.dtype == W.BF16 else torch.float16
    conv = (lambda a: torch.from_numpy(a).view(view).to(dev)) if w.dtype == W.BF16 else \
        (lambda a: torch.from_numpy(a).to(dev))
    return conv(w.q), conv(w.k_pool), conv(w.v_pool)


def time_kernel(pk, p, copies, iters, warmup=10):
    """run() durations (ms) on the stream it launches on, cycling through the
    input copies (so every launch reads inputs no earlier launch has left in
    the caches): `warmup` untimed launches, then `iters` launches each
    bracketed by its own pair of HIP events.  Returns (mean, median, bracket):
    bracket is one event pair around the same number of back-to-back launches
    divided by their count (no per-launch event packets between them)."""
    import torch
    s = torch.cuda.current_stream()
    q0 = copies[0][0]
    o = torch.empty((p.total_q_rows, p.num_qo_heads, p.head_dim), dtype=p.dtype, device=q0.device)
    lse = torch.empty((p.total_q_rows, p.num_qo_heads), dtype=torch.float32, device=q0.device)
    for i in range(warmup):
        p.run(*copies[i % len(copies)], out=o, lse=lse)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for i, (a, b) in enumerate(evs):
        a.record(s)
        p.run(*copies[i % len(copies)], out=o, lse=lse)
        b.record(s)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs])
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    for i in range(iters):
        p.run(*copies[i % len(copies)], out=o, lse=lse)
    b.record(s)
    torch.cuda.synchronize()
    return float(per.mean()), float(np.median(per)), a.elapsed_time(b) / iters


def rotation_copies(tensors, touched_bytes, min_touched=512_000_000, max_copies=16):
    """Device copies of (q, k, v) so that at least `min_touched` bytes of
    inputs are read between two launches that use the same copy (the 256 MB
    Infinity Cache then holds none of a launch's inputs)."""
    n = max(1, min(max_copies, -(-min_touched // max(touched_bytes, 1))))
    out = [tuple(tensors)]
    for _ in range(n - 1):
        out.append(tuple(t.clone() for t in tensors))
    return out


def plan_cost_us(pk, w, dt, dev, reps=50, **opts):
    """Host cost of planning this workload, median over `reps` calls (us):
    'c_abi' is pkv_plan alone through the C ABI (validation, scheduling and the
    task-list upload launch; workspaces already allocated), 'python' is the
    binding's plan() (sizing, two workspace allocations, pkv_plan)."""
    import ctypes
    import torch
    lib = pk.load_library()
    p0 = pk.plan(**w.plan_args(), dtype=dt, device=dev, **opts)
    int_ws, float_ws = p0._int_ws, p0._float_ws
    a = w.plan_args()
    qo, kv, idx, last, batch = pk._plan_arrays(a["qo_indptr"], a["kv_indptr"],
                                               a["kv_page_indices"], a["kv_last_page_len"])
    o = pk._options(**{k: v for k, v in a.items() if k in ("custom_mask", "mask_indptr",
                                                          "logits_soft_cap")}, **opts)
    code = pk._dtype_code(dt)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    args = (pk._ptr_i32(qo), pk._ptr_i32(kv), pk._ptr_i32(idx), len(idx), pk._ptr_i32(last),
            batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, int(w.causal),
            w.window_left, ctypes.c_float(w.sm_scale), code, int_ws.data_ptr(), int_ws.numel(),
            float_ws.data_ptr(), float_ws.numel() * 4, stream, ctypes.byref(o))
    h = ctypes.c_void_p()
    c_times, py_times = [], []
    torch.cuda.synchronize()
    for i in range(reps + 5):
        t0 = time.perf_counter()
        st = lib.pkv_plan(*args, ctypes.byref(h))
        t1 = time.perf_counter()
        assert st == 0, lib.pkv_last_error()
        lib.pkv_plan_destroy(h)
        if i >= 5:
            c_times.append((t1 - t0) * 1e6)
    for i in range(reps + 5):
        t0 = time.perf_counter()
        pk.plan(**w.plan_args(), dtype=dt, device=dev, **opts)
        t1 = time.perf_counter()
        if i >= 5:
            py_times.append((t1 - t0) * 1e6)
    torch.cuda.synchronize()
    return {"c_abi": float(np.median(c_times)), "python": float(np.median(py_times))}


def copy_ceiling(torch, dev, nbytes=1 << 30, iters=10):
    """HBM GB/s of a device-to-device copy (bytes read + bytes written)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(iters):
        dst.copy_(src)
    b.record(s)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    del src, dst
    torch.cuda.empty_cache()
    gbs = 2 * nbytes / ms / 1e6
    return {"GB/s": gbs, "frac": gbs / PEAK_HBM_GBS, "bytes": 2 * nbytes}


def cpu_baseline(w, min_s=10.0, budget_s=20.0):
    """The float64 oracle on the workload's requests (cheapest first), in whole
    passes repeated until at least min_s of work, stopping mid-pass past budget_s."""
    import oracle
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         "unknown")
    except OSError:  # pragma: no cover
        pass
    qf, kf, vf = w.float_inputs()
    order = np.argsort(w.qo_lens * w.kv_lens)   # cheapest requests first
    jobs = []   # (request, q slice, oracle arguments, flops)
    for b in order:
        sub = W.Workload(**{**w.__dict__,
                            "qo_lens": w.qo_lens[b:b + 1], "kv_lens": w.kv_lens[b:b + 1],
                            "qo_indptr": np.array([0, w.qo_lens[b]], np.int32),
                            "kv_indptr": np.array([0, w.kv_indptr[b + 1] - w.kv_indptr[b]], np.int32),
                            "kv_page_indices": w.kv_page_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]],
                            "kv_last_page_len": w.kv_last_page_len[b:b + 1]})
        a = sub.plan_args()
        del a["head_dim"]
        jobs.append((int(b), slice(int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])), a,
                     attention_flops(sub)))
    passes, partial, flops, t0 = 0, [], 0.0, time.perf_counter()
    while True:
        partial = []
        for b, qs, a, f in jobs:
            oracle.attention(qf[qs], kf, vf, **a)
            partial.append(b)
            flops += f
            if time.perf_counter() - t0 > budget_s:
                break
        if len(partial) == len(jobs):
            passes, partial = passes + 1, []
        dt = time.perf_counter() - t0
        if dt >= min_s or partial:
            break
    what = f"{passes} whole pass{'es' if passes != 1 else ''} over all {w.batch_size} requests"
    if partial:
        what += f" and requests {sorted(partial)} of one more"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": model, "blas": blas, "blas_threads": int(threads),
            "sample": f"float64 numpy oracle, {what}, all {w.num_qo_heads} q heads, {dt:.1f} s; "
                      f"host has {os.cpu_count()} logical CPUs"}


def _random_pools(w, dev, copies, seed, kv_fp8=False):
    """Timing-only pools of the workload's shape: N(0, 1) drawn on the device
    (as E4M3 codes for FP8 caches)."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    dt = torch.bfloat16 if w.dtype == W.BF16 else torch.float16
    kdt = torch.float8_e4m3fn if kv_fp8 else dt
    shape = (w.num_pages, w.page_size, w.num_kv_heads, w.head_dim)
    mk = lambda: torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(kdt)
    q = torch.randn((w.total_q, w.num_qo_heads, w.head_dim), generator=g, device=dev,
                    dtype=torch.float32).to(dt)
    return q, [(mk(), mk()) for _ in range(copies)]


def time_rotating(p, q, pools, iters, warmup=2):
    """Average run() time (ms) from HIP events, cycling through K/V pool copies.

    Returns (eager, graph): eager brackets each run() call on the stream, so it
    includes the host's per-call cost whenever that exceeds the kernels'; graph
    replays one captured HIP graph holding one run() per pool copy and divides
    by the copies, which is the device time of the launches alone (run() makes
    no allocation, copy or synchronisation, so it can be captured)."""
    import torch
    s = torch.cuda.current_stream()
    o = torch.empty((p.total_q_rows, p.num_qo_heads, p.head_dim), dtype=p.dtype, device=q.device)
    lse = torch.empty((p.total_q_rows, p.num_qo_heads), dtype=torch.float32, device=q.device)
    for i in range(warmup):
        k, v = pools[i % len(pools)]
        p.run(q, k, v, out=o, lse=lse)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for i, (a, b) in enumerate(evs):
        k, v = pools[i % len(pools)]
        a.record(s)
        p.run(q, k, v, out=o, lse=lse)
        b.record(s)
    torch.cuda.synchronize()
    eager = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k, v in pools:
            p.run(q, k, v, out=o, lse=lse)
    g.replay()
    torch.cuda.synchronize()
    reps = max(2, iters // len(pools))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(s)
        g.replay()
        b.record(s)
    torch.cuda.synchronize()
    graph = float(np.mean([a.elapsed_time(b) for a, b in evs])) / len(pools)
    del g
    return eager, graph


def coverage(pk, torch, dev, iters=20):
    """Every workload of the path, each against the roofline that binds it:
    workloads above the ridge point (peak flops / peak bytes, about 312 flop per
    byte) report algorithmic TFLOP/s against the bf16 MFMA peak, the others
    (verify, decode over long contexts, narrow windows) algorithmic GB/s (K/V
    rows any query row can see, plus q, o, lse) against the HBM peak.  K/V pools rotate so that at least 512 MB is touched
    between reuses of a pool (the 256 MB Infinity Cache cannot hold them)."""
    rows = []
    for i, (name, w, opts) in enumerate(coverage_cases()):
        dt = torch.bfloat16 if w.dtype == W.BF16 else torch.float16
        kv_fp8 = opts.get("kv_dtype") == "fp8_e4m3"
        nbytes = kv_bytes(w, 1 if kv_fp8 else 2)
        copies = max(1, min(16, -(-512_000_000 // max(nbytes, 1))))
        q, pools = _random_pools(w, dev, copies, seed=7000 + i, kv_fp8=kv_fp8)
        p = pk.plan(**w.plan_args(), dtype=dt, device=dev, **opts)
        eager_ms, ms = time_rotating(p, q, pools, iters)
        flops = attention_flops(w)
        # the roofline that binds: arithmetic intensity against the ridge point
        hbm_bound = flops / nbytes < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
        rec = {"workload": name, "ms": ms, "eager_ms": eager_ms, "TFLOP/s": flops / ms / 1e9,
               "GB/s": nbytes / ms / 1e6, "bound": "hbm" if hbm_bound else "mfma",
               "pool_copies": copies, "work_items": p.info["num_work_items"],
               "split_tiles": p.info["num_merge_items"]}
        rec["frac"] = rec["GB/s"] / PEAK_HBM_GBS if hbm_bound else rec["TFLOP/s"] / PEAK_BF16_TFLOPS
        rec["plan_us"] = plan_cost_us(pk, w, dt, dev, **opts)
        rows.append(rec)
        del q, pools, p
        torch.cuda.empty_cache()
    for name, w, per_req in (("append_prefill_b8", W.config2(values=False), None),
                             ("append_verify_b64_hkv8", W.config4(batch=64, values=False), 4)):
        rows.append(time_append(pk, torch, dev, name, w, per_req, iters))
    rows.append(time_sampling(pk, torch, dev, iters))
    return rows


def coverage_cases():
    """(name, workload without values, plan options) of every timed workload."""
    cases = [("single_contiguous_w-1", W.config1(values=False), {}),
             ("single_contiguous_w31", W.config1(window_left=31, values=False), {}),
             ("paged_prefill_b8_w127", W.config2(window_left=127, values=False), {})]
    for page in (1024, 16):
        for wl in (0, 31, 127, 8192):
            cases.append((f"noncausal_window_b4_p{page}_w{wl}",
                          W.config3(window_left=wl, page_size=page, values=False), {}))
    for b in (4, 16, 64):
        for h in (4, 8):
            cases.append((f"verify_b{b}_hkv{h}", W.config4(batch=b, num_kv_heads=h, values=False), {}))
    for b in (16, 64):
        cases.append((f"tree_verify_b{b}_hkv8_8nodes", W.tree_verify(batch=b, values=False), {}))
    capped = W.config2(values=False)
    capped.logits_soft_cap = 50.0
    cases.append(("paged_prefill_b8_softcap50", capped, {}))
    rng = np.random.default_rng(2560)
    qo = rng.integers(128, 1024, size=4, endpoint=True)
    kv = qo + rng.integers(0, 2048, size=4, endpoint=True)
    cases.append(("prefill_d256_b4_hq16_hkv8", W.build("prefill_d256", qo, kv, 16, 8, 256, 16, True,
                                                      -1, W.BF16, seed=None, rng=rng, values=False), {}))
    kv_v = rng.integers(512, 8192, size=16, endpoint=True)
    cases.append(("verify_d256_b16_hq16_hkv8", W.build("verify_d256", [4] * 16, kv_v, 16, 8, 256, 16,
                                                      True, -1, W.BF16, seed=None, rng=rng,
                                                      values=False), {}))
    fp8 = {"kv_dtype": "fp8_e4m3", "k_scale": 0.5, "v_scale": 2.0}
    cases.append(("verify_b64_hkv8_fp8kv", W.config4(batch=64, values=False), fp8))
    cases.append(("paged_prefill_b8_fp8kv", W.config2(values=False), fp8))
    # FP8 caches under a topology mask, and under a soft-cap
    cases.append(("tree_verify_b16_hkv8_8nodes_fp8kv", W.tree_verify(batch=16, values=False), fp8))
    capped8 = W.config2(values=False)
    capped8.logits_soft_cap = 50.0
    cases.append(("paged_prefill_b8_softcap50_fp8kv", capped8, fp8))
    for ql in (1, 64):
        for wl in (-1, 4095):
            cases.append((f"long_ctx_q{ql}_w{wl}_8chunks",
                          W.config5(qo_len=ql, window_left=wl, values=False),
                          {"num_kv_chunks": W.CONFIG5_CHUNKS}))
    return cases


def time_sampling(pk, torch, dev, iters):
    """chain_speculative_sampling over 64 requests x 4 drafts x a 128256-entry
    vocabulary.  Algorithmic bytes: per draft position examined, its token's
    two probabilities and its uniform; the row the draw reads (target and draft
    rows at a rejection, the bonus target row otherwise); the outputs."""
    inp = W.spec_sampling_inputs()
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in inp.items()}
    B, n = inp["draft_token_ids"].shape
    V = inp["target_probs"].shape[2]
    args = (t["draft_probs"], t["draft_token_ids"], t["target_probs"], t["accept_u"],
            t["sample_u"])
    ws = torch.empty(pk.load_library().pkv_chain_speculative_sampling_workspace_size(B, V),
                     dtype=torch.uint8, device=dev)
    out, acc = pk.chain_speculative_sampling(*args, workspace=ws)
    torch.cuda.synchronize()
    acc_h = acc.cpu().numpy().astype(np.int64)
    examined = np.minimum(acc_h + 1, n)
    nbytes = int((examined * 12).sum() + ((acc_h < n) * 8 * V + (acc_h == n) * 4 * V).sum()
                 + B * (4 * (n + 1) + 8))
    # copies of the probability arrays, taken in turn, so that the rows the
    # calls read between two uses of one copy (4 x ~66 MB) exceed the 256 MB
    # Infinity Cache
    ncopy = 5
    copies = [args] + [(args[0].clone(), args[1], args[2].clone(), args[3], args[4])
                       for _ in range(ncopy - 1)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in copies:
            pk.chain_speculative_sampling(*c, out=out, num_accepted=acc, workspace=ws)
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(2, iters // ncopy))]
    for a, b in evs:
        a.record(s)
        g.replay()
        b.record(s)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs])) / ncopy
    del g, t, copies
    torch.cuda.empty_cache()
    return {"workload": "spec_sampling_b64_n4_v128256", "ms": ms, "GB/s": nbytes / ms / 1e6,
            "bound": "hbm", "frac": nbytes / ms / 1e6 / PEAK_HBM_GBS,
            "mean_accepted": float(acc_h.mean()), "input_copies": ncopy}


def time_append(pk, torch, dev, name, w, per_req, iters):
    """append_kv of the workload's last `per_req` keys per request (all keys when
    None) into its paged pools.  Algorithmic bytes: the new K and V rows read
    once and written once, plus 8 bytes of (request, position) per token."""
    dt = torch.bfloat16 if w.dtype == W.BF16 else torch.float16
    bi, pos = [], []
    for b in range(w.batch_size):
        L = int(w.kv_lens[b])
        n = L if per_req is None else min(per_req, L)
        bi.append(np.full(n, b, np.int32))
        pos.append(np.arange(L - n, L, dtype=np.int32))
    bi = torch.from_numpy(np.concatenate(bi)).to(dev)
    pos = torch.from_numpy(np.concatenate(pos)).to(dev)
    tokens = bi.numel()
    indptr = torch.from_numpy(w.kv_indptr.astype(np.int32)).to(dev)
    pages = torch.from_numpy(w.kv_page_indices.astype(np.int32)).to(dev)
    shape = (w.num_pages, w.page_size, w.num_kv_heads, w.head_dim)
    k = torch.zeros(shape, dtype=dt, device=dev)
    v = torch.zeros(shape, dtype=dt, device=dev)
    row_bytes = w.num_kv_heads * w.head_dim * 2
    nbytes = tokens * (4 * row_bytes + 8)
    copies = max(1, min(8, -(-512_000_000 // max(2 * tokens * row_bytes, 1))))
    srcs = [(torch.randn((tokens, w.num_kv_heads, w.head_dim), device=dev).to(dt),
             torch.randn((tokens, w.num_kv_heads, w.head_dim), device=dev).to(dt))
            for _ in range(copies)]
    s = torch.cuda.current_stream()
    for i in range(2):
        pk.append_kv(*srcs[i % copies], bi, pos, indptr, pages, k, v)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()       # device time of the launches (see time_rotating)
    with torch.cuda.graph(g):
        for src in srcs:
            pk.append_kv(*src, bi, pos, indptr, pages, k, v)
    g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(2, iters // copies))]
    for a, b in evs:
        a.record(s)
        g.replay()
        b.record(s)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs])) / copies
    del g
    rec = {"workload": name, "ms": ms, "GB/s": nbytes / ms / 1e6, "bound": "hbm",
           "tokens": tokens, "source_copies": copies}
    rec["frac"] = rec["GB/s"] / PEAK_HBM_GBS
    del srcs, k, v
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--window-left", type=int, default=-1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-coverage", action="store_true",
                    help="skip timing the other workloads against their rooflines")
    ap.add_argument("--kernel-iters", type=int, default=50)
    ap.add_argument("--profile", action="store_true",
                    help="short run for profilers: 3 steps, 1 warmup, no baselines")
    ap.add_argument("--profile-verify", action="store_true",
                    help="short run for profilers of the verify workload instead (batch 64, "
                         "Hkv 8): 5 launches, one JSON line with its algorithmic bytes")
    ap.add_argument("--profile-case", default=None,
                    help="short run for profilers of one timed workload by name (see "
                         "coverage_cases): 5 launches over rotating pools, one JSON line with "
                         "its algorithmic bytes and flops")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 256 MiB read + 256 MiB write elementwise kernel "
                         "(scale for the HBM byte counters)")
    args = ap.parse_args()
    if args.profile:
        args.steps, args.warmup, args.kernel_iters = 3, 1, 3
        args.no_cpu_baseline = args.no_coverage = True
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged-KV prefill path has no multi-GPU "
              "component here (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_prefill_amd as pk
    pk.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calib_copy:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)       # 256 MiB read, 256 MiB written
        torch.cuda.synchronize()
        del src, dst

    if args.profile_case:
        found = [c for c in coverage_cases() if c[0] == args.profile_case]
        if not found:
            print(f"unknown workload {args.profile_case!r}; known: "
                  f"{[c[0] for c in coverage_cases()]}", file=sys.stderr)
            sys.exit(2)
        name, w, opts = found[0]
        kv_fp8 = opts.get("kv_dtype") == "fp8_e4m3"
        nbytes = kv_bytes(w, 1 if kv_fp8 else 2)
        ncopy = max(1, min(16, -(-512_000_000 // max(nbytes, 1))))
        q, pools = _random_pools(w, dev, ncopy, seed=9100, kv_fp8=kv_fp8)
        dt = torch.bfloat16 if w.dtype == W.BF16 else torch.float16
        p = pk.plan(**w.plan_args(), dtype=dt, device=dev, **opts)
        ms, _ = time_rotating(p, q, pools, 5, warmup=1)
        print(json.dumps({"workload": name, "algorithmic_bytes_per_launch": nbytes,
                          "algorithmic_flops_per_launch": attention_flops(w),
                          "work_items": p.info["num_work_items"],
                          "split_tiles": p.info["num_merge_items"], "eager_ms": ms}))
        return

    if args.profile_verify:
        w = W.config4(batch=64, num_kv_heads=8, values=False)
        q, pools = _random_pools(w, dev, 1, seed=7064)
        p = pk.plan(**w.plan_args(), dtype=torch.bfloat16, device=dev)
        ms, _ = time_rotating(p, q, pools, 5, warmup=1)
        print(json.dumps({"workload": "verify_b64_hkv8",
                          "kv_bytes_per_launch": kv_bytes(w), "eager_ms": ms}))
        return

    w = W.config2(window_left=args.window_left)
    # copies of the inputs, cycled so that >= 512 MB of inputs is read between
    # two uses of one copy (the Infinity Cache cannot serve a step's inputs)
    copies = rotation_copies(_device_inputs(w, dev), kv_bytes(w))
    plan_args = w.plan_args()
    flops = attention_flops(w)

    def step(i):
        p = pk.plan(**plan_args, dtype=torch.bfloat16, device=dev)
        p.run(*copies[i % len(copies)])
        return p

    for i in range(args.warmup):
        p = step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        p = step(args.warmup + i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt / args.steps * 1e3
    value = flops / (dt / args.steps) / 1e12

    kernel_ms, kernel_median_ms, kernel_bracket_ms = time_kernel(
        pk, p, copies, max(50, args.kernel_iters) if not args.profile else args.kernel_iters)
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch_size,
                   "qo_len": "U[128,1024]", "kv_len": "qo + U[0,2048]", "page_size": w.page_size,
                   "num_qo_heads": w.num_qo_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "causal": w.causal, "window_left": w.window_left,
                   "total_q": w.total_q, "flops_per_step": flops,
                   "input_copies": len(copies)},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(),
                     "kernel": "attn_kernel (prefill tile)", "kernel_ms": kernel_ms,
                     "kernel_median_ms": kernel_median_ms,
                     "kernel_bracket_ms": kernel_bracket_ms,
                     "frac_median": flops / (kernel_median_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "plan_us": plan_cost_us(pk, w, torch.bfloat16, dev) if not args.profile else None,
    }
    if not args.no_coverage:
        result["coverage"] = coverage(pk, torch, dev)
        result["copy_ceiling"] = copy_ceiling(torch, dev)
        # the short-query verify kernel against the HBM roofline (its largest batch)
        v = next(r for r in result["coverage"] if r["workload"] == "verify_b64_hkv8")
        result["roofline_verify"] = {
            "bound": "hbm", "achieved": v["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": v["GB/s"] / PEAK_HBM_GBS, "traffic": measured_traffic(VERIFY_TRAFFIC_FILE),
            "kernel": "attn_kernel (short-query tile)", "workload": "verify_b64_hkv8",
            "kernel_ms": v["ms"]}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
