"""Benchmark: ragged MLA prefill on one MI355X.

Headline: the DeepSeek-V3-shaped ragged batch (16 sequences, lengths drawn
uniformly in [256, 4096], 128 heads, bf16 Q/K dim 192, V dim 128, causal,
seed 2). One step = one pass of the hot path over that batch:
  plan the work list on the host from the indptrs, upload it (async copy on
  the stream), run the prefill kernel (O and LSE).
Inputs are resident in HBM before the timed region. The step is timed with
a barrier + torch.cuda.synchronize() on both sides; the kernel alone is
timed with HIP events recorded on the stream it is launched on.

FLOPs = 2 * heads * (visible query-key pairs) * (192 + 128) (algorithmic:
masked work inside partial tiles is not counted).

Also measured in the same run (reported under "secondary"): merge_state at
the chunked-prefill size (16384 tokens x 128 heads, bf16), against the HBM
roofline; the device-planned path, the chunked prefill with its merges, the
paged context pass, a skewed batch, KV decompression followed by prefill,
and the weight-absorbed prefill over the latent cache.

cpu_baseline: the fp64 oracle (test infrastructure, timed as it stands) on a
bounded sample of the same workload's (row, head) pairs, on this host's cores.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import math
import os
import random
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz (published: 2.5 PFLOP/s dense)
PEAK_HBM_GBS = 8000.0         # HBM3E, 8 TB/s
PEAK_FP32_TFLOPS = 157.3       # fp32 dense MFMA (published)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def visible_pairs(qo, kv, causal):
    n = 0
    for b in range(len(qo) - 1):
        ql, kl = qo[b + 1] - qo[b], kv[b + 1] - kv[b]
        if not causal:
            n += ql * kl
            continue
        for_rows = 0
        # rows i see min(kl, max(0, kl - ql + i + 1)) keys
        for i in range(ql):
            for_rows += min(kl, max(0, kl - ql + i + 1))
        n += for_rows
    return n


def code_hash(path):
    """sha256 (16 hex) of a source file's code with comments and blank lines removed."""
    import hashlib
    import re
    txt = open(path).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    lines = [l.split("//")[0].strip() for l in txt.splitlines()]
    return hashlib.sha256("\n".join(l for l in lines if l).encode()).hexdigest()[:16]


def profile_traffic(profile, source):
    """HBM bytes per launch from a committed counter profile, or None when the
    profile is missing or the kernel's code changed since it was taken."""
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("source_code_sha256_16") != code_hash(os.path.join(ROOT, source)):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def device_info(torch):
    """What the peaks are set against: the device's name and CU count as the
    runtime reports them; the peaks themselves are MI355X's published ones."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "peak_basis": "bf16 dense 256 CU x 4096 flop/clk x 2.4 GHz; HBM3E 8 TB/s"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time for the oracle baseline sample (0 = skip)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--n-xcd", type=int, default=8)
    ap.add_argument("--only", choices=["merge", "decompress", "absorbed", "decode", "fp32",
                                       "skewed", "fused"],
                    default=None,
                    help="run only one secondary kernel (for profiling) and print its figures")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times) and exit; "
                         "its FETCH_SIZE / WRITE_SIZE counters calibrate the traffic figures")
    return ap.parse_args()


def time_prefill(mra, torch, x, steps, warmup, n_xcd):
    plan = mra.Plan(n_xcd=n_xcd)
    out = torch.empty((x.q.shape[0], x.num_heads, 128), dtype=x.q.dtype, device=x.q.device)
    lse = torch.empty((x.q.shape[0], x.num_heads), dtype=torch.float32, device=x.q.device)

    plan_s = []

    def step(ev=None):
        t = time.perf_counter()
        plan.plan(x.qo_indptr, x.kv_indptr, x.num_heads, x.causal, x.q.dtype)
        plan_s.append(time.perf_counter() - t)
        # (the upload may wait for a staging slot whose copy is still queued
        # behind earlier kernels: GPU back-pressure, not planning work)
        plan.upload()
        if ev is not None:
            ev[0].record()
        plan.run(x.q, x.k, x.v, x.sm_scale, out=out, lse=lse)
        if ev is not None:
            ev[1].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    plan_s.clear()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    info = plan.info()
    info["plan_ms"] = sum(plan_s) / len(plan_s) * 1e3
    return wall, kern_ms, info


def cpu_baseline(oracle, torch, x, target_s, seed=0):
    """Oracle TFLOP/s on a random sample of (row, head) pairs of the workload."""
    rng = random.Random(seed)
    qo, kv = x.qo_indptr, x.kv_indptr
    heads = sorted(rng.sample(range(x.num_heads), min(2, x.num_heads)))
    host = {h: (x.q[:, h:h + 1].contiguous().cpu(), x.k[:, h:h + 1].contiguous().cpu(),
                x.v[:, h:h + 1].contiguous().cpu()) for h in heads}

    def keys_seen(t):
        b = max(i for i in range(len(qo) - 1) if qo[i] <= t)
        ql, kl = qo[b + 1] - qo[b], kv[b + 1] - kv[b]
        i = t - qo[b]
        return kl if not x.causal else min(kl, max(0, kl - ql + i + 1))

    def run(n_rows):
        rows = sorted(rng.randrange(qo[-1]) for _ in range(n_rows))
        pairs = sum(keys_seen(t) for t in rows) * len(heads)
        t0 = time.perf_counter()
        for h in heads:
            q, k, v = host[h]
            oracle.prefill(q, k, v, qo, kv, x.causal, x.sm_scale, rows)
        return time.perf_counter() - t0, pairs, n_rows

    dt, pairs, n = run(64)
    n2 = max(64, min(200000, int(64 * target_s / max(dt, 1e-3))))
    dt, pairs, n = run(n2)
    flops = 2.0 * pairs * 320
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "nproc": os.cpu_count(), "cpu_model": cpu_model,
            "kind": "oracle",
            "sample": f"{n} random query rows x {len(heads)} heads (heads {heads}) of the same "
                      f"batch, {pairs} visible pairs, {dt:.1f} s, fp64"}


def _keys_seen(qo, kv, causal, t):
    b = max(i for i in range(len(qo) - 1) if qo[i] <= t)
    ql, kl = qo[b + 1] - qo[b], kv[b + 1] - kv[b]
    i = t - qo[b]
    return kl if not causal else min(kl, max(0, kl - ql + i + 1))


def _cpu_note(oracle):
    return {"cores": oracle.num_threads(), "nproc": os.cpu_count(), "kind": "oracle"}


def oracle_sampled(oracle, torch, q, k, v, qo, kv, causal, sm_scale, num_heads, target_s,
                   seed, extra_pairs_per_row=None, run_fn=None):
    """Oracle wall time on seeded random query rows of one head, extrapolated
    linearly in visible (row, key) pairs to every row and every head."""
    rng = random.Random(seed)
    h = rng.randrange(num_heads)
    host = (q[:, h:h + 1].contiguous().cpu(), k[:, h:h + 1].contiguous().cpu(),
            v[:, h:h + 1].contiguous().cpu())
    total_pairs = visible_pairs(qo, kv, causal)

    def run(n_rows):
        rows = sorted(set(rng.randrange(qo[-1]) for _ in range(n_rows)))
        pairs = sum(_keys_seen(qo, kv, causal, t) for t in rows)
        if extra_pairs_per_row is not None:
            pairs += extra_pairs_per_row * len(rows)
        t0 = time.perf_counter()
        if run_fn is not None:
            run_fn(h, host, rows)
        else:
            oracle.prefill(*host, qo, kv, causal, sm_scale, rows)
        return time.perf_counter() - t0, pairs, len(rows)

    if run_fn is not None:
        run_fn(h, host, [qo[-1] - 1])   # untimed: one-time set-up inside run_fn
    dt, pairs, n = run(32)
    n2 = max(32, min(100000, int(32 * target_s / max(dt, 1e-3))))
    dt, pairs, n = run(n2)
    if extra_pairs_per_row is not None:
        total_pairs += extra_pairs_per_row * qo[-1]
    full_s = dt * (total_pairs * num_heads) / max(pairs, 1)
    out = {"sample": f"{n} seeded random query rows of head {h} (seed {seed}), {pairs} "
                     f"visible pairs, fp64", "sample_s": round(dt, 3),
           "sample_frac_of_work": pairs / (total_pairs * num_heads),
           "extrapolated_full_s": round(full_s, 2),
           "extrapolated": "linear in visible (row, key) pairs over every row and head"}
    out.update(_cpu_note(oracle))
    return out


def oracle_tiny_full(oracle, torch, workloads):
    """The tiny fp32 workload through the oracle in full, next to the GPU call."""
    import mla_ragged_chunked_amd as mra
    x = workloads.tiny_fp32()
    t0 = time.perf_counter()
    oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, x.causal, x.sm_scale)
    cpu_s = time.perf_counter() - t0
    g = [t.cuda() for t in (x.q, x.k, x.v)]
    mra.ragged_prefill(*g, x.qo_indptr, x.kv_indptr, x.causal, x.sm_scale)
    torch.cuda.synchronize()
    ts = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        mra.ragged_prefill(*g, x.qo_indptr, x.kv_indptr, x.causal, x.sm_scale)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    out = {"workload": "tiny_fp32: lengths 1, 17, 64, 4 heads, fp32, causal",
           "oracle_full_s": round(cpu_s, 5), "gpu_call_ms": round(sorted(ts)[10], 4)}
    out.update(_cpu_note(oracle))
    return out


def time_merge(mra, torch, workloads, steps, warmup):
    tokens, heads = 16384, 128
    o_a, l_a, o_b, l_b = workloads.merge_inputs(tokens, heads, torch.bfloat16, seed=43,
                                                device="cuda")
    out = torch.empty_like(o_a)
    out_l = torch.empty_like(l_a)
    for _ in range(warmup):
        mra.merge_state(o_a, l_a, o_b, l_b, out=out, out_lse=out_l)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        mra.merge_state(o_a, l_a, o_b, l_b, out=out, out_lse=out_l)
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    rows = tokens * heads
    bytes_ = rows * (3 * 128 * 2 + 3 * 4)      # read o_a, o_b, lse_a, lse_b; write o, lse
    gbs = bytes_ / (ms * 1e-3) / 1e9
    # a plain device-to-device copy of the same byte count, as a measured ceiling
    src = torch.empty(bytes_ // 2, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(steps):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() / (c0.elapsed_time(c1) / steps * 1e-3) / 1e9
    del src, dst
    return {"workload": f"merge_state {tokens} tokens x {heads} heads, bf16",
            "kernel_ms": round(ms, 4), "GB/s": round(gbs, 1),
            "device_copy_GB/s": round(copy_gbs, 1), "frac_of_copy": round(gbs / copy_gbs, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": profile_traffic("merge_state_16384x128_bf16.txt",
                                                    "mla_ragged_chunked_amd/csrc/merge.hip")}}


def time_chunked(mra, torch, workloads, steps, warmup):
    """Chunked prefill pipeline: one causal pass over the new tokens, one
    non-causal pass per context chunk, then merge_state folds the partials."""
    c = workloads.chunked_prefill(device="cuda")
    m = c.main
    plans = [mra.Plan().plan(ch.qo_indptr, ch.kv_indptr, ch.num_heads, False).upload()
             for ch in c.chunks]
    plans.append(mra.Plan().plan(m.qo_indptr, m.kv_indptr, m.num_heads, True).upload())
    passes = [(p, ch) for p, ch in zip(plans, c.chunks + [m])]
    outs = [(torch.empty((m.q.shape[0], m.num_heads, 128), dtype=m.q.dtype, device="cuda"),
             torch.empty((m.q.shape[0], m.num_heads), dtype=torch.float32, device="cuda"))
            for _ in passes]
    fo, fl = torch.empty_like(outs[0][0]), torch.empty_like(outs[0][1])

    # HIP events between the stages: 3 passes, then 2 merges
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        for i, ((p, x), (o, l)) in enumerate(zip(passes, outs)):
            p.run(x.q, x.k, x.v, x.sm_scale, out=o, lse=l)
            if ev is not None:
                ev[1 + i].record()
        mra.merge_state(outs[0][0], outs[0][1], outs[1][0], outs[1][1], out=fo, out_lse=fl)
        if ev is not None:
            ev[4].record()
        mra.merge_state(fo, fl, outs[2][0], outs[2][1], out=fo, out_lse=fl)
        if ev is not None:
            ev[5].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    stage = [sum(e[k].elapsed_time(e[k + 1]) for e in evs) / steps for k in range(5)]
    pairs = sum(visible_pairs(x.qo_indptr, x.kv_indptr, x.causal) for x in c.chunks + [m])
    flops = 2.0 * m.num_heads * pairs * 320
    return {"workload": "chunked_prefill: 8 x (2048 new causal + 2 x 4096 context), 128 heads, "
                        "3 prefill passes + 2 merge_state",
            "ms_per_step": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 1),
            "flops_per_step": flops,
            "context_pass_ms": [round(stage[0], 4), round(stage[1], 4)],
            "new_token_pass_ms": round(stage[2], 4),
            "passes_ms": round(stage[0] + stage[1] + stage[2], 4),
            "merges_ms": round(stage[3] + stage[4], 4)}


def time_paged_context(mra, torch, workloads, steps, warmup, page=64):
    """One chunked-prefill context pass (8 x 2048 new tokens against 8 x 4096
    context keys, non-causal) with the context in a page pool in random page
    order, next to the same pass on contiguous K/V. Both through the one-shot
    calls (each includes its host planning)."""
    c = workloads.chunked_prefill(device="cuda")
    ch = c.chunks[0]
    tk, heads = ch.k.shape[0], ch.num_heads
    n_pages = tk // page
    g = torch.Generator(device="cuda").manual_seed(3)
    perm = torch.randperm(n_pages, generator=g, device="cuda")
    kc = torch.empty((n_pages, page, heads, 192), dtype=ch.k.dtype, device="cuda")
    vc = torch.empty((n_pages, page, heads, 128), dtype=ch.v.dtype, device="cuda")
    kc.index_copy_(0, perm, ch.k.view(n_pages, page, heads, 192))
    vc.index_copy_(0, perm, ch.v.view(n_pages, page, heads, 128))
    lens = [b - a for a, b in zip(ch.kv_indptr, ch.kv_indptr[1:])]
    per = max(n // page for n in lens)
    table = perm.view(len(lens), per).to(torch.int32).contiguous()
    out = torch.empty((ch.q.shape[0], heads, 128), dtype=ch.q.dtype, device="cuda")
    lse = torch.empty((ch.q.shape[0], heads), dtype=torch.float32, device="cuda")

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3

    contig = timed(lambda: mra.ragged_prefill(ch.q, ch.k, ch.v, ch.qo_indptr, ch.kv_indptr, False,
                                              ch.sm_scale, out=out, lse=lse))
    paged = timed(lambda: mra.ragged_prefill_paged(ch.q, kc, vc, ch.qo_indptr, ch.kv_indptr,
                                                   table, False, ch.sm_scale, out=out, lse=lse))
    flops = 2.0 * heads * visible_pairs(ch.qo_indptr, ch.kv_indptr, False) * 320
    return {"workload": f"context pass 8 x (2048 queries x 4096 keys), 128 heads, pages of {page} "
                        "in random order",
            "contiguous_ms": round(contig, 4), "paged_ms": round(paged, 4),
            "contiguous_TFLOP/s": round(flops / contig / 1e9, 1),
            "paged_TFLOP/s": round(flops / paged / 1e9, 1)}


def time_workload_prefill(mra, torch, x, steps, warmup, name):
    plan = mra.Plan().plan(x.qo_indptr, x.kv_indptr, x.num_heads, x.causal, x.q.dtype).upload()
    out = torch.empty((x.q.shape[0], x.num_heads, 128), dtype=x.q.dtype, device="cuda")
    lse = torch.empty((x.q.shape[0], x.num_heads), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        plan.run(x.q, x.k, x.v, x.sm_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        plan.run(x.q, x.k, x.v, x.sm_scale, out=out, lse=lse)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2.0 * x.num_heads * visible_pairs(x.qo_indptr, x.kv_indptr, x.causal) * 320
    return {"workload": name, "kernel_ms": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 1),
            "flops": flops}


def time_fp32_prefill(mra, torch, workloads, steps, warmup):
    """The fp32 path (fp32 matrix-core kernel, no bf16 rounding) on the
    DeepSeek-V3 lengths at 16 heads, against the fp32 dense MFMA peak."""
    lens = workloads.deepseek_v3_lengths(2)
    x = workloads.ragged_inputs(lens, lens, 16, torch.float32, seed=2, causal=True,
                                device="cuda")
    r = time_workload_prefill(mra, torch, x, steps, warmup,
                              "deepseek_v3_batch lengths at 16 heads, fp32 inputs and outputs")
    r["roofline"] = {"bound": "mfma", "achieved": r["TFLOP/s"], "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(r["TFLOP/s"] / PEAK_FP32_TFLOPS, 4),
                     "traffic": profile_traffic("prefill_fp32_deepseek_v3_lengths_16heads.txt",
                                                "mla_ragged_chunked_amd/csrc/prefill_fp32.hip"),
                     "kernel": "prefill_fp32_kernel"}
    return r


def time_device_plan(mra, torch, x, steps, warmup):
    """The same batch through the device-planned path (device indptrs, work
    list built on the GPU, no host sync): eager, and replayed from a captured
    graph. Times cover the planning kernels and the prefill."""
    batch = len(x.qo_indptr) - 1
    tq, tk = x.qo_indptr[-1], x.kv_indptr[-1]
    dp = mra.DevicePlan(batch, tq, tk, x.num_heads, x.q.dtype)
    qo_d = torch.tensor(x.qo_indptr, dtype=torch.int32, device="cuda")
    kv_d = torch.tensor(x.kv_indptr, dtype=torch.int32, device="cuda")
    out = torch.empty((tq, x.num_heads, 128), dtype=x.q.dtype, device="cuda")
    lse = torch.empty((tq, x.num_heads), dtype=torch.float32, device="cuda")
    run = lambda: dp.run(x.q, x.k, x.v, qo_d, kv_d, x.causal, x.sm_scale, out=out, lse=lse)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / steps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / steps
    flops = 2.0 * x.num_heads * visible_pairs(x.qo_indptr, x.kv_indptr, x.causal) * 320
    return {"workload": "deepseek_v3_batch through the device-planned path",
            "eager_ms": round(eager_ms, 4), "eager_TFLOP/s": round(flops / eager_ms / 1e9, 1),
            "graph_replay_ms": round(graph_ms, 4),
            "graph_TFLOP/s": round(flops / graph_ms / 1e9, 1),
            "invalid_flag": int(dp.invalid_flag().item())}


def time_decompress(mra, torch, workloads, steps, warmup, with_prefill=True):
    d = workloads.decompress_batch(device="cuda")
    H = d.num_heads
    k, v = mra.decompress_kv(d.c_kv, d.k_rope, d.w_uk, d.w_uv, H)
    for _ in range(warmup):
        mra.decompress_kv(d.c_kv, d.k_rope, d.w_uk, d.w_uv, H, k_out=k, v_out=v)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        mra.decompress_kv(d.c_kv, d.k_rope, d.w_uk, d.w_uv, H, k_out=k, v_out=v)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    t = d.c_kv.shape[0]
    gemm_flops = 2.0 * 2 * t * 512 * H * 128
    # algorithmic bytes: c_kv, k_rope and both weights read once, K and V written once
    algo_bytes = 2.0 * (t * 512 + t * 64 + 2 * 512 * H * 128 + t * H * (192 + 128))
    tflops = gemm_flops / ms / 1e9
    out = {"workload": "decompress_batch: 8 x 4096 tokens, latent 512 -> 128 heads (K_nope, V), "
                       "then causal prefill",
           "decompress_ms": round(ms, 4), "decompress_TFLOP/s": round(tflops, 1),
           "decompress_GB/s": round(algo_bytes / ms / 1e6, 1),
           "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                        "hbm_frac": round(algo_bytes / ms / 1e6 / PEAK_HBM_GBS, 4),
                        "traffic": profile_traffic("decompress_kv_8x4096_128heads.txt",
                                                   "mla_ragged_chunked_amd/csrc/decompress.hip"),
                        "kernel": "decompress_kernel"}}
    if not with_prefill:
        return out
    x = workloads.PrefillInputs(d.q, k, v, d.indptr, d.indptr, H, True, d.sm_scale)
    pre = time_workload_prefill(mra, torch, x, steps, warmup, "prefill on the decompressed K/V")
    out.update({"prefill_ms": pre["kernel_ms"], "prefill_TFLOP/s": pre["TFLOP/s"],
                "end_to_end_ms": round(ms + pre["kernel_ms"], 4)})
    return out


def fused_key_tiles(qo, kv, causal, block_m=128, block_n=32):
    """32-key tiles the fused kernel decompresses per head: every 128-row
    query tile decompresses each key tile it visits."""
    n = 0
    for b in range(len(qo) - 1):
        ql, kl = qo[b + 1] - qo[b], kv[b + 1] - kv[b]
        for r0 in range(0, ql, block_m):
            rows = min(block_m, ql - r0)
            hi = min(kl, max(0, kl - ql + r0 + rows)) if causal else kl
            n += -(-hi // block_n)
    return n


def time_fused_decompress(mra, torch, workloads, steps, warmup, extras=True):
    """Decompression fused into the prefill on the decompression workload
    (8 x 4096 tokens, 128 heads, causal), and the absorbed kernel on the same
    lengths. The fused kernel's MFMA work is the attention plus the
    decompression of every key tile once per query tile that visits it."""
    d = workloads.decompress_batch(device="cuda")
    H = d.num_heads
    o, lse = mra.decompress_prefill(d.q, d.c_kv, d.k_rope, d.w_uk, d.w_uv, d.indptr, d.indptr,
                                    True, d.sm_scale)
    args = (d.q, d.c_kv, d.k_rope, d.w_uk, d.w_uv, d.indptr, d.indptr, True, d.sm_scale)
    for _ in range(warmup):
        mra.decompress_prefill(*args, out=o, lse=lse)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        mra.decompress_prefill(*args, out=o, lse=lse)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = visible_pairs(d.indptr, d.indptr, True)
    attn_flops = 2.0 * H * pairs * 320
    tiles = fused_key_tiles(d.indptr, d.indptr, True)
    dec_flops = 2.0 * 2 * 32 * 512 * 128 * tiles * H
    mfma = (attn_flops + dec_flops) / ms / 1e9
    fused = {"fused_ms": round(ms, 4),
             "attention_TFLOP/s": round(attn_flops / ms / 1e9, 1),
             "decompressed_key_tiles_per_head": tiles,
             "mfma_flop": attn_flops + dec_flops,
             "roofline": {"bound": "mfma", "achieved": round(mfma, 1), "peak": PEAK_BF16_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(mfma / PEAK_BF16_TFLOPS, 4),
                          "traffic": profile_traffic("decompress_prefill_fused_8x4096_128heads.txt",
                                                     "mla_ragged_chunked_amd/csrc/decompress_prefill.hip"),
                          "kernel": "decompress_prefill_kernel"}}
    del o, lse, d
    torch.cuda.empty_cache()
    if not extras:
        return fused, None
    # the absorbed kernel on the same lengths (its query and output projections,
    # Q_nope W_UK^T and O_latent W_UV, are extra GEMMs outside this kernel)
    lens = [4096] * 8
    x = workloads.absorbed_inputs(lens, lens, H, seed=6, causal=True, device="cuda")
    out, alse = mra.absorbed_prefill(x.q, x.kv, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    for _ in range(warmup):
        mra.absorbed_prefill(x.q, x.kv, x.qo_indptr, x.kv_indptr, True, x.sm_scale, out=out,
                             lse=alse)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        mra.absorbed_prefill(x.q, x.kv, x.qo_indptr, x.kv_indptr, True, x.sm_scale, out=out,
                             lse=alse)
    e1.record()
    torch.cuda.synchronize()
    ams = e0.elapsed_time(e1) / steps
    aflops = 2.0 * H * pairs * (576 + 512)
    absorbed = {"absorbed_ms": round(ams, 4), "absorbed_TFLOP/s": round(aflops / ams / 1e9, 1),
                "projection_flop_outside_kernel": 2.0 * 2 * x.q.shape[0] * H * 128 * 512}
    del out, alse, x
    torch.cuda.empty_cache()
    fused["short_chunks"] = time_fused_short_chunks(mra, torch, workloads, steps, warmup)
    return fused, absorbed


def time_fused_short_chunks(mra, torch, workloads, steps, warmup, n_req=16, new=128,
                            prefix=4096, H=128):
    """Where each key tile is visited by one query tile only: n_req requests
    of `new` query tokens over their own `prefix` + `new` keys (bottom-right
    causal). The two-call path decompresses every key token to HBM and then
    runs the prefill; the fused kernel decompresses each key tile once on chip."""
    x = workloads.latent_prefill_inputs([new] * n_req, [prefix + new] * n_req, H, seed=13,
                                        causal=True, device="cuda")
    tk = x.c_kv.shape[0]

    def timed(fn):
        fn()
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    o = torch.empty((x.q.shape[0], H, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((x.q.shape[0], H), dtype=torch.float32, device="cuda")
    fused_ms = timed(lambda: mra.decompress_prefill(x.q, x.c_kv, x.k_rope, x.w_uk, x.w_uv,
                                                    x.qo_indptr, x.kv_indptr, True, x.sm_scale,
                                                    out=o, lse=lse))
    k = torch.empty((tk, H, 192), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((tk, H, 128), dtype=torch.bfloat16, device="cuda")
    dec_ms = timed(lambda: mra.decompress_kv(x.c_kv, x.k_rope, x.w_uk, x.w_uv, H, k_out=k,
                                             v_out=v))
    pre_ms = timed(lambda: mra.ragged_prefill(x.q, k, v, x.qo_indptr, x.kv_indptr, True,
                                              x.sm_scale, out=o, lse=lse))
    del x, o, lse, k, v
    torch.cuda.empty_cache()
    return {"workload": f"{n_req} requests x {new} new tokens over {prefix} + {new} keys, "
                        f"{H} heads, causal",
            "fused_ms": round(fused_ms, 4), "two_call_decompress_ms": round(dec_ms, 4),
            "two_call_prefill_ms": round(pre_ms, 4),
            "two_call_end_to_end_ms": round(dec_ms + pre_ms, 4)}


def time_absorbed(mra, torch, workloads, steps, warmup):
    """Weight-absorbed prefill over the latent cache on the DeepSeek-V3 batch
    lengths: 576-dim absorbed queries, 576-dim shared cache rows, 512-dim
    values, 128 heads, causal. FLOPs = 2 * heads * visible pairs * (576 + 512)."""
    x = workloads.absorbed_batch(device="cuda")
    H = x.num_heads
    pairs = visible_pairs(x.qo_indptr, x.kv_indptr, x.causal)
    flops = 2.0 * H * pairs * (576 + 512)
    out, lse = mra.absorbed_prefill(x.q, x.kv, x.qo_indptr, x.kv_indptr, x.causal, x.sm_scale)
    for _ in range(warmup):
        mra.absorbed_prefill(x.q, x.kv, x.qo_indptr, x.kv_indptr, x.causal, x.sm_scale,
                             out=out, lse=lse)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        mra.absorbed_prefill(x.q, x.kv, x.qo_indptr, x.kv_indptr, x.causal, x.sm_scale,
                             out=out, lse=lse)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tflops = flops / ms / 1e9
    # the same rows from a page pool (pages of 64 in a seeded random order)
    page = 64
    lens = [b - a for a, b in zip(x.kv_indptr, x.kv_indptr[1:])]
    per = [-(-n // page) for n in lens]
    g = torch.Generator().manual_seed(11)
    perm = torch.randperm(sum(per), generator=g).tolist()
    pool = torch.empty((sum(per), page, 576), dtype=x.kv.dtype, device="cuda")
    table = torch.zeros((len(lens), max(per)), dtype=torch.int32)
    i = 0
    for b, n in enumerate(lens):
        for pg in range(per[b]):
            table[b, pg] = perm[i]
            m = min(page, n - pg * page)
            pool[perm[i], :m] = x.kv[x.kv_indptr[b] + pg * page:x.kv_indptr[b] + pg * page + m]
            i += 1
    table = table.to("cuda")
    po, pl = mra.absorbed_prefill_paged(x.q, pool, x.qo_indptr, x.kv_indptr, table, x.causal,
                                        x.sm_scale)
    torch.cuda.synchronize()
    same = bool(torch.equal(po, out) and torch.equal(pl, lse))
    e0.record()
    for _ in range(steps):
        mra.absorbed_prefill_paged(x.q, pool, x.qo_indptr, x.kv_indptr, table, x.causal,
                                   x.sm_scale, out=po, lse=pl)
    e1.record()
    torch.cuda.synchronize()
    ms_paged = e0.elapsed_time(e1) / steps
    del pool, po, pl
    return {"workload": f"absorbed_batch: DeepSeek-V3 batch lengths, {x.qo_indptr[-1]} tokens, "
                        f"{H} heads, q [T,H,576] over kv [T,576], Dv 512, causal",
            "kernel_ms": round(ms, 4), "TFLOP/s": round(tflops, 1), "flops": flops,
            "paged_kernel_ms": round(ms_paged, 4),
            "paged_TFLOP/s": round(flops / ms_paged / 1e9, 1),
            "paged_bit_identical": same,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": profile_traffic(
                             "prefill_absorbed_deepseek_v3_batch.txt",
                             "mla_ragged_chunked_amd/csrc/prefill_absorbed.hip"),
                         "kernel": "prefill_absorbed_kernel"}}


def time_absorbed_decode(mra, torch, workloads, steps, warmup, batch=64, prefix=4096):
    """One decode step through the absorbed path: `batch` requests, one new
    token each, over `prefix`-token latent caches, 128 heads. Each cache row is
    read once for all heads (algorithmic bytes: q, kv, out, lse once); at 128
    heads that is ~240 flop per byte, so the HBM floor of the step is only a
    little above its MFMA floor and both fractions are reported."""
    x = workloads.absorbed_inputs([1] * batch, [prefix] * batch, 128, seed=53, causal=True,
                                  device="cuda")
    H = x.num_heads
    pairs = visible_pairs(x.qo_indptr, x.kv_indptr, x.causal)
    flops = 2.0 * H * pairs * (576 + 512)
    nbytes = 2.0 * (batch * H * 576 + batch * prefix * 576 + batch * H * 512) + 4.0 * batch * H
    # planned once, run per layer (the plan/run split); the one-shot call,
    # which plans on the host every time, is timed next to it
    plan = mra.AbsorbedPlan().plan(x.qo_indptr, x.kv_indptr, H, True).upload()
    splits = plan.info()["kv_splits"]
    out, lse = plan.run(x.q, x.kv, x.sm_scale)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(lambda: plan.run(x.q, x.kv, x.sm_scale, out=out, lse=lse))
    ms_one_shot = timed(lambda: mra.absorbed_prefill(x.q, x.kv, x.qo_indptr, x.kv_indptr, True,
                                                     x.sm_scale, out=out, lse=lse))
    gbs = nbytes / ms / 1e6
    return {"workload": f"absorbed decode: {batch} requests x 1 token over {prefix}-token latent "
                        f"caches, {H} heads, bf16",
            "step_ms": round(ms, 4), "one_shot_ms": round(ms_one_shot, 4), "kv_splits": splits,
            "TFLOP/s": round(flops / ms / 1e9, 1), "GB/s": round(gbs, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "mfma_frac": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                         "note": "step = one run of a plan made once: the absorbed kernel "
                                 "and the KV-split merge; the HBM floor is the larger one, "
                                 "but the MFMA floor is close (all heads share a cache row)"}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    import mla_ragged_chunked_amd as mra
    import workloads

    torch.cuda.set_device(0)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes 3 times (read {n} B + write {n} B per copy)")
        return
    mra.lib()
    if args.only == "merge":
        print(json.dumps(time_merge(mra, torch, workloads, args.steps, args.warmup)), flush=True)
        return
    if args.only == "decode":
        print(json.dumps(time_absorbed_decode(mra, torch, workloads, args.steps, args.warmup)),
              flush=True)
        return
    if args.only == "absorbed":
        print(json.dumps(time_absorbed(mra, torch, workloads, args.steps, args.warmup)), flush=True)
        return
    if args.only == "decompress":
        print(json.dumps(time_decompress(mra, torch, workloads, args.steps, args.warmup,
                                         with_prefill=False)), flush=True)
        return
    if args.only == "fused":
        # the fused kernel on the decompression workload alone (for profiling)
        fused, _ = time_fused_decompress(mra, torch, workloads, args.steps, args.warmup,
                                         extras=False)
        print(json.dumps(fused), flush=True)
        return
    if args.only == "skewed":
        xs = workloads.skewed_batch(device="cuda")
        r = time_workload_prefill(
            mra, torch, xs, args.steps, args.warmup,
            f"skewed_batch: 64 log-uniform lengths [16, 32768], {xs.qo_indptr[-1]} tokens, 128 heads")
        r["seq_lens"] = [xs.qo_indptr[i + 1] - xs.qo_indptr[i] for i in range(len(xs.qo_indptr) - 1)]
        print(json.dumps(r), flush=True)
        return
    if args.only == "fp32":
        print(json.dumps(time_fp32_prefill(mra, torch, workloads, args.steps, args.warmup)),
              flush=True)
        return
    t0 = time.perf_counter()
    x = workloads.deepseek_v3_batch(device="cuda")
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s: T={x.qo_indptr[-1]} H={x.num_heads}")
    pairs = visible_pairs(x.qo_indptr, x.kv_indptr, x.causal)
    flops = 2.0 * x.num_heads * pairs * (192 + 128)

    wall, kern_ms, info = time_prefill(mra, torch, x, args.steps, args.warmup, args.n_xcd)
    ms_step = wall / args.steps * 1e3
    k_ms = sum(kern_ms) / len(kern_ms)
    value = flops * args.steps / wall / 1e12
    achieved = flops / (k_ms * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms, kernel {k_ms:.3f} ms ({achieved:.1f} TFLOP/s), "
        f"{info['n_items']} work items")

    result = {
        "metric": "ragged MLA prefill TFLOP/s (bf16, Dqk192/Dvo128) and % of MFMA peak, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, DeepSeek-V3 MLA prefill shapes)",
        "config": {"workload": "deepseek_v3_batch", "num_seqs": x.batch,
                   "tokens": x.qo_indptr[-1], "heads": x.num_heads, "dqk": 192, "dvo": 128,
                   "causal": True, "sm_scale": x.sm_scale, "seed": 2,
                   "seq_lens": [b - a for a, b in zip(x.qo_indptr, x.qo_indptr[1:])],
                   "visible_pairs_per_head": pairs, "flops_per_step": flops,
                   "work_items": info["n_items"], "block_m": info["block_m"],
                   "n_xcd": info["n_xcd"]},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": profile_traffic("prefill_bf16_deepseek_v3_batch.txt",
                                                "mla_ragged_chunked_amd/csrc/prefill_bf16.hip"),
                     "kernel": "prefill_bf16_kernel",
                     "kernel_ms": round(k_ms, 4),
                     "kernel_ms_median": round(sorted(kern_ms)[len(kern_ms) // 2], 4),
                     "host_plan_ms": round(info["plan_ms"], 4)},
        "device": device_info(torch),
    }
    if args.cpu_seconds > 0:
        import oracle
        log("timing the oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(oracle, torch, x, args.cpu_seconds)
    if not args.no_secondary:
        sec = {"merge_state": time_merge(mra, torch, workloads, args.steps, args.warmup)}
        log("secondary: device-planned path ...")
        sec["device_plan"] = time_device_plan(mra, torch, x, args.steps, args.warmup)
        del x
        torch.cuda.empty_cache()
        log("secondary: one GPU's share of an 8-way head split ...")
        xh = workloads.deepseek_v3_batch(device="cuda", num_heads=16)
        sec["head_shard_h16"] = time_workload_prefill(
            mra, torch, xh, args.steps, 1,
            "deepseek_v3_batch at 16 heads: one GPU's share when its 128 heads are split "
            "over 8 GPUs (same sequences, same kernel)")
        del xh
        torch.cuda.empty_cache()
        log("secondary: chunked prefill ...")
        sec["chunked_prefill"] = time_chunked(mra, torch, workloads, max(3, args.steps // 4), 1)
        if args.cpu_seconds > 0:
            import oracle
            log("oracle: chunked prefill sample ...")
            c = workloads.chunked_prefill(device="cuda")
            m = c.main

            def run_chunked(h, host, rows):
                kvs = [(ch.k[:, h:h + 1].contiguous().cpu(), ch.v[:, h:h + 1].contiguous().cpu(),
                        ch.kv_indptr) for ch in c.chunks]
                oracle.chunked(host[0], host[1], host[2], m.qo_indptr, kvs, m.sm_scale, rows)

            ctx_per_row = sum(ch.kv_indptr[-1] for ch in c.chunks) // len(c.chunks[0].kv_indptr[:-1])
            sec["chunked_prefill"]["cpu_oracle"] = oracle_sampled(
                oracle, torch, m.q, m.k, m.v, m.qo_indptr, m.kv_indptr, True, m.sm_scale,
                m.num_heads, args.cpu_seconds / 3, seed=3, extra_pairs_per_row=ctx_per_row,
                run_fn=run_chunked)
            del c, m
        torch.cuda.empty_cache()
        log("secondary: paged context pass ...")
        sec["paged_context"] = time_paged_context(mra, torch, workloads, max(3, args.steps // 4), 1)
        torch.cuda.empty_cache()
        log("secondary: skewed batch ...")
        xs = workloads.skewed_batch(device="cuda")
        sec["skewed_batch"] = time_workload_prefill(
            mra, torch, xs, max(3, args.steps // 4), 1,
            f"skewed_batch: 64 log-uniform lengths [16, 32768], {xs.qo_indptr[-1]} tokens, 128 heads")
        # the lengths after the 262,144-token cap rule, as drawn
        sec["skewed_batch"]["seq_lens"] = [xs.qo_indptr[i + 1] - xs.qo_indptr[i]
                                           for i in range(len(xs.qo_indptr) - 1)]
        if args.cpu_seconds > 0:
            import oracle
            log("oracle: skewed batch sample ...")
            sec["skewed_batch"]["cpu_oracle"] = oracle_sampled(
                oracle, torch, xs.q, xs.k, xs.v, xs.qo_indptr, xs.kv_indptr, True, xs.sm_scale,
                xs.num_heads, args.cpu_seconds / 3, seed=4)
        del xs
        torch.cuda.empty_cache()
        log("secondary: decompression + prefill ...")
        sec["decompress_batch"] = time_decompress(mra, torch, workloads, max(3, args.steps // 4), 1)
        if args.cpu_seconds > 0:
            import oracle
            log("oracle: decompression + prefill sample ...")
            d = workloads.decompress_batch(device="cuda")
            c_kv, k_rope = d.c_kv.cpu(), d.k_rope.cpu()
            dec = {}

            def run_dec(h, host, rows):
                # the decompression of head h (every token) is timed once and
                # kept; each sample then times the prefill rows alone
                if h not in dec:
                    t0 = time.perf_counter()
                    wk = d.w_uk[:, h * 128:(h + 1) * 128].contiguous().cpu()
                    wv = d.w_uv[:, h * 128:(h + 1) * 128].contiguous().cpu()
                    rk, rv = oracle.decompress(c_kv, k_rope, wk, wv, 1)
                    dec[h] = (rk, rv, time.perf_counter() - t0)
                rk, rv, _ = dec[h]
                oracle.prefill(host[0].double(), rk, rv, d.indptr, d.indptr, True, d.sm_scale, rows)

            # K and V stand in for the decompressed ones (only their shapes are used)
            r = oracle_sampled(oracle, torch, d.q, d.q, d.q[:, :, :128], d.indptr, d.indptr,
                               True, d.sm_scale, d.num_heads, args.cpu_seconds / 3, seed=5,
                               run_fn=run_dec)
            dec_s = next(iter(dec.values()))[2]
            r["decompress_one_head_s"] = round(dec_s, 3)
            r["extrapolated_full_s"] = round(r["extrapolated_full_s"] + dec_s * d.num_heads, 2)
            r["extrapolated"] = ("prefill linear in visible (row, key) pairs over every row and "
                                 "head, plus the one-head decompression time x heads")
            sec["decompress_batch"]["cpu_oracle"] = r
            del d, c_kv, k_rope
        torch.cuda.empty_cache()
        log("secondary: decompression fused into the prefill ...")
        fused, absorbed = time_fused_decompress(mra, torch, workloads, max(3, args.steps // 4), 1)
        sec["decompress_batch"]["fused"] = fused
        sec["decompress_batch"]["absorbed_same_lengths"] = absorbed
        log("secondary: absorbed prefill over the latent cache ...")
        sec["absorbed_batch"] = time_absorbed(mra, torch, workloads, max(3, args.steps // 4), 1)
        torch.cuda.empty_cache()
        log("secondary: absorbed decode step ...")
        sec["absorbed_decode"] = time_absorbed_decode(mra, torch, workloads, args.steps, 2)
        torch.cuda.empty_cache()
        log("secondary: fp32 prefill ...")
        sec["fp32_prefill"] = time_fp32_prefill(mra, torch, workloads, max(3, args.steps // 4), 1)
        torch.cuda.empty_cache()
        if args.cpu_seconds > 0:
            import oracle
            sec["tiny_fp32"] = oracle_tiny_full(oracle, torch, workloads)
        result["secondary"] = sec
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
