"""MLA decode throughput on one MI355X: cached tokens attended per second.

One step = mla_decode (query projection from h with W^DQ, W^UQ, absorption
with W^UK, split-KV attention over the latent cache) + mla_combine (split
merge and W^UV) for every sequence of the batch, on a cache that
mla_cache_append built beforehand.  Inputs are seeded synthetic data at the
DeepSeek-V3 MLA shape; several copies of cache and weights are rotated from
step to step so that no step finds its data in the 256 MB last-level cache.

Prints ONE JSON line (see --help).  The dominant kernel is the split-KV
attention (mla_decode_attend): its duration is taken with HIP events around
that call on the stream it runs on, inside the timed region.  A timing event
holds the stream for a few microseconds (it waits for the work before it to
drain), so the events bracket the phases of every n-th timed step only
(n = steps // 64, at least 1) and the other steps run back to back.
"""
import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode cached-tokens/s + % HBM/MFMA roofline, B=64 L=4096 bf16, 1 GPU"
HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # dense bf16 flop/s, MI355X


def algorithmic(spec, dims, lengths):
    """Algorithmic bytes and flops of one step and of one attention launch."""
    H, dh, dr, dc, dq, d = (dims[k] for k in ("n_heads", "d_head", "d_rope", "d_c", "d_cq", "d_model"))
    s_q = spec["s_q"]
    fp8_tok = dc + 4 * (dc // 128) + 2 * dr
    tok_bytes = {"bf16": (dc + dr) * 2, "fp8": fp8_tok, "fp8e8": fp8_tok, "f32": (dc + dr) * 4}[spec["cache"]]
    es = 2 if spec["act"] == "bf16" else 4
    L = [int(x) for x in lengths]
    vis = sum(max(0, Lb - s_q + j + 1) for Lb in L for j in range(s_q))
    cache = sum(L) * tok_bytes
    attn_flops = vis * H * 2 * ((dc + dr) + dc)
    R = len(L) * s_q
    if spec.get("weights") == "fp8":  # E4M3 codes and one fp32 scale per 128 x 128 block
        w_el = dq * d + H * (dh + dr) * dq + 2 * H * dh * dc
        w_bytes = w_el + 4 * w_el // (128 * 128)
    else:
        w_bytes = es * (dq * d + H * (dh + dr) * dq + 2 * H * dh * dc)
    io_bytes = es * (R * d + R * H * dh)
    q_flops = 2 * R * (dq * d + H * (dh + dr) * dq + H * dh * dc)
    o_flops = 2 * R * H * dh * dc
    return dict(step_bytes=cache + w_bytes + io_bytes, step_flops=attn_flops + q_flops + o_flops,
                attn_bytes=cache, attn_flops=attn_flops)


# Sources that define the attention kernel of each cache type; a traffic
# figure measured with hardware counters is reported only while they are
# unchanged since the measurement.
ATTN_SOURCES = {"bf16": ["fast_attn2.hip", "layout.hpp", "common.hpp"],
                "fp8": ["fast_attn2.hip", "layout.hpp", "common.hpp"],
                "fp8e8": ["fast_attn2.hip", "layout.hpp", "common.hpp"],
                "prefill": ["fast_prefill.hip", "internal.hpp", "common.hpp"]}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")
MTP_ACCEPTANCE = 0.85  # second-token acceptance of MTP drafts, lower end of the pages' 85-90%


def attn_source_sha(cache):
    h = hashlib.sha256()
    for f in ATTN_SOURCES.get(cache, []):
        with open(os.path.join(ROOT, "mla_latent_kv_29_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, cache, splits=None):
    """HBM bytes per attention launch from the committed counter measurement
    (FETCH_SIZE + WRITE_SIZE scaled by a plain copy of known size), or None if
    there is none for this workload, the kernel changed since, or it was taken
    at another split count (the partial rows written depend on it)."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_sha256") != attn_source_sha(cache):
        return None
    if splits is not None and rec.get("splits", splits) != splits:
        return None
    return rec.get("hbm_bytes_per_launch")


def record_traffic(workload, fetch_csv, write_csv):
    """Writes the HBM traffic of the workload's attention kernel into the
    traffic record: the two counter files are `rocprofv3 --pmc FETCH_SIZE`
    and `--pmc WRITE_SIZE` runs of `bench.py --workload W --steps 3 --warmup 1
    --no-cpu-baseline --copy-calibration 1024`.  Each counter is averaged per
    dispatch of the attention kernel and scaled by what it reads for the
    plain copy of 1024 MiB (torch.neg over fp32) in the same run."""
    import csv
    from mla_latent_kv_29_amd import inputs
    prefill = workload in inputs.PREFILL_WORKLOADS
    cache = "prefill" if prefill else inputs.WORKLOADS[workload]["cache"]
    key = "k_prefill_attn" if prefill else "k_attn_v3b"

    def per_dispatch(path, counter):
        vals = {"attn": {}, "copy": {}}
        with open(path, newline="") as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                kind = "attn" if key in row["Kernel_Name"] else "copy" if "neg_kernel_cuda" in row["Kernel_Name"] \
                    else None
                if kind:
                    d = vals[kind]
                    d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
        if not vals["attn"] or not vals["copy"]:
            raise SystemExit(f"{path}: no {key} or copy dispatch with {counter}")
        return (sum(vals["attn"].values()) / len(vals["attn"]), sum(vals["copy"].values()) / len(vals["copy"]))

    splits = None
    if not prefill:  # the split count the counter runs used: the session's plan for the workload's lengths
        from mla_latent_kv_29_amd import _lib as L
        spec = inputs.WORKLOADS[workload]
        dims = spec["dims"]
        lengths = inputs.seqlens(spec["lengths"], spec["batch"], 0, spec["index"])
        table, _ = inputs.block_table(lengths, dims["page_size"], spec["table"], 0, spec["index"])
        cd = L.make_dims(dims)
        plan = L.mla_plan_splits(cd, spec["batch"], spec["s_q"], table.shape[1], lengths)
        splits = L.mla_decode_splits(cd, spec["batch"], spec["s_q"], table.shape[1], plan)
    fa, fc = per_dispatch(fetch_csv, "FETCH_SIZE")
    wa, wc = per_dispatch(write_csv, "WRITE_SIZE")
    copy_bytes = 1024 * 1024 * 1024
    fscale, wscale = copy_bytes / (fc * 1024), copy_bytes / (wc * 1024)
    cmd = ("cd /tmp && rocprofv3 --pmc {c} --output-format csv -d <out> -o run -- python3 /root/repo/bench.py "
           f"--workload {workload} --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration 1024")
    rec = {"kernel_source_sha256": attn_source_sha(cache), "sources": ATTN_SOURCES[cache], "splits": splits,
           "fetch_kib_per_dispatch": fa, "write_kib_per_dispatch": wa, "copy_fetch_kib": fc, "copy_write_kib": wc,
           "copy_bytes_each_way": copy_bytes, "fetch_scale": fscale, "write_scale": wscale,
           "hbm_bytes_per_launch": fa * 1024 * fscale + wa * 1024 * wscale,
           "command_fetch": cmd.format(c="FETCH_SIZE"), "command_write": cmd.format(c="WRITE_SIZE")}
    try:
        with open(TRAFFIC_FILE) as fh:
            allrec = json.load(fh)
    except (OSError, ValueError):
        allrec = {}
    allrec[workload] = rec
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(allrec, fh, indent=1)
        fh.write("\n")
    print(json.dumps({"workload": workload, "hbm_bytes_per_launch": rec["hbm_bytes_per_launch"],
                      "fetch_scale": fscale, "write_scale": wscale}))


def cpu_baseline(spec, dims, W, gen_h, lengths, budget_s, max_seqs=64):
    """The float64 oracle (decode from cached latents, explicit per-head k^C and
    v^C) on a bounded sample of sequences of the same workload; cached
    tokens/s = sum of sample lengths / oracle time."""
    import numpy as np
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = None
    Wn = {k: v.to("cpu", torch.float64).numpy() for k, v in W.items()}
    s_q = spec["s_q"]
    fp8w = spec.get("weights") == "fp8"
    if fp8w:  # the weights' block quantisation is preparation, not part of a step: untimed
        Wq = {k: oracle.quantize_blocks(Wn[k]) for k in ("W_DQ", "W_UQ", "W_UK", "W_UV")}
    order = np.argsort(lengths)[::-1] if spec["lengths"][0] != "fixed" else range(len(lengths))
    t_used, toks, n = 0.0, 0, 0
    for b in list(order)[:max_seqs]:
        Lb = int(lengths[b])
        h = gen_h(int(b), 0, Lb).to("cpu", torch.float64).numpy()
        c, kr = oracle.kv_latents(h, Wn["W_DKV"], Wn["W_KR"], np.arange(Lb), dims["rope_theta"])
        hq = h[Lb - s_q:Lb]
        tau = 1.0 / math.sqrt(dims["d_head"] + dims["d_rope"])
        t0 = time.perf_counter()
        if fp8w:
            oracle.decode_fp8w_from_latents(c, kr, hq, Wq, dims, Lb, s_q, tau)
        else:
            oracle.decode_from_latents(c, kr, hq, Wn["W_DQ"], Wn["W_UQ"], Wn["W_UK"], Wn["W_UV"], dims, Lb, s_q, tau)
        t_used += time.perf_counter() - t0
        toks += Lb
        n += 1
        if t_used >= budget_s:
            break
    return {"value": toks / t_used, "unit": "cached-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} sequence(s), {toks} cached tokens, float64 numpy, decode from cached latents "
                      + ("(FP8 block-scaled projections, absorbed form)" if fp8w else
                         "(explicit k^C/v^C per head)") + f", {t_used:.1f} s",
            "host_cpus": os.cpu_count(), "cpu_model": platform.processor() or platform.machine()}


def prefill_algorithmic(dims, lengths):
    """FLOPs of one prefill: the causal attention (query-key pairs with
    t <= j, q.k over d_head + d_rope and p.v over d_head, per head) and the
    projections (c^KV, k^R, c^Q, q, k^C, v^C)."""
    H, dh, dr, dc, dq, d = (dims[k] for k in ("n_heads", "d_head", "d_rope", "d_c", "d_cq", "d_model"))
    L = [int(x) for x in lengths]
    n = sum(L)
    pairs = sum(x * (x + 1) // 2 for x in L)
    attn = pairs * H * 2 * ((dh + dr) + dh)
    proj = 2 * n * (dc * d + dr * d + dq * d + H * (dh + dr) * dq + 2 * H * dh * dc)
    return attn, proj


def copy_calibration(mib, dev):
    """A plain elementwise copy of `mib` MiB (read once, written once), run
    three times untimed: the known-size reference that scales the hardware
    byte counters of a profiled run."""
    if mib <= 0:
        return
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def run_hbm_probe(args):
    """Achievable HBM bandwidth on this GPU: a plain streaming read
    (mla_hbm_read_probe: 16-byte loads over the whole GPU) and a copy
    (torch's copy kernel), each over several buffers in turn so that no pass
    finds its data in the 256 MB last-level cache; 75 MB and 302 MB (one
    attention launch's query rows and cache).  Reports the median over the
    passes."""
    import numpy as np
    import torch
    from mla_latent_kv_29_amd import _lib as L
    torch.cuda.set_device(0)
    dev = "cuda:0"
    props = torch.cuda.get_device_properties(0)
    res = {"probe": "hbm", "device": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
           "compute_units": props.multi_processor_count, "results": []}
    for mb in (75, 302):
        n = mb * 1000 * 1000 // 4
        nbuf = max(2, (1024 // mb) + 1)
        srcs = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(nbuf)]
        dsts = [torch.empty_like(srcs[0]) for _ in range(nbuf)]
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        for kind in ("read", "copy"):
            ts = []
            for rep in range(3 * nbuf + 20):
                i = rep % nbuf
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                if kind == "read":
                    L.mla_hbm_read_probe(srcs[i], 4 * n, sink)
                else:
                    dsts[i].copy_(srcs[i])
                e1.record()
                e1.synchronize()
                if rep >= nbuf:
                    ts.append(e0.elapsed_time(e1) * 1e-3)
            t = float(np.median(ts))
            moved = 4 * n * (1 if kind == "read" else 2)
            res["results"].append({"kind": kind, "mb": mb, "us": t * 1e6, "GB_per_s": moved / t / 1e9,
                                   "bytes": moved})
        del srcs, dsts
        torch.cuda.empty_cache()
    print(json.dumps(res))


class PowerSampler:
    """Board power and mean shader clock from `amd-smi metric -p -c`, sampled
    in a background thread: [(time, watts, MHz)]."""

    def __init__(self):
        import threading
        self.samples, self.stop, self.ok = [], False, True
        self.th = threading.Thread(target=self.run, daemon=True)
        self.th.start()

    def run(self):
        import re
        import subprocess
        while not self.stop:
            t = time.time()
            try:
                out = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c"], capture_output=True, text=True,
                                     timeout=10).stdout
            except (OSError, subprocess.SubprocessError):
                self.ok = False
                return
            pw = re.search(r"SOCKET_POWER:\s*(\d+)\s*W", out)
            clks = [int(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", out)]
            if pw:
                self.samples.append((t, int(pw.group(1)), sum(clks) / len(clks) if clks else None))
            time.sleep(0.05)

    def mean(self, t0, t1):
        s = [x for x in self.samples if t0 <= x[0] <= t1]
        if not s:
            return None, None, 0
        c = [x[2] for x in s if x[2] is not None]
        return sum(x[1] for x in s) / len(s), (sum(c) / len(c) if c else None), len(s)


def run_mfma_probe(secs):
    """Achievable bf16 MFMA rate: the register-
    only MFMA probe (mla_mfma_probe, 4096 waves of v_mfma_f32_32x32x16_bf16
    chains) launched back to back for `secs` seconds while amd-smi samples
    power and clocks; the rate is taken over the whole window (launch time
    from the wall clock), after 2 s of warm-up launches."""
    import torch
    from mla_latent_kv_29_amd import _lib as L
    torch.cuda.set_device(0)
    dev = "cuda:0"
    g = torch.Generator(device="cpu").manual_seed(7)
    ops = torch.randn(12 * 64 * 8, generator=g).to(torch.bfloat16).to(dev)
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    iters = 2000
    ps = PowerSampler()
    time.sleep(1.0)
    t0 = time.time()
    time.sleep(2.0)
    idle = ps.mean(t0 + 0.3, time.time())
    _, flops = L.mla_mfma_probe(ops, iters, sink)
    t0 = time.time()
    while time.time() - t0 < 2.0:
        for _ in range(20):
            L.mla_mfma_probe(ops, iters, sink)
        torch.cuda.synchronize()
    n, t0 = 0, time.time()
    while time.time() - t0 < secs:
        for _ in range(20):
            L.mla_mfma_probe(ops, iters, sink)
        n += 20
        torch.cuda.synchronize()
    t1 = time.time()
    ps.stop = True
    p, clk, ns = ps.mean(t0 + 0.3, t1)
    launch_s = (t1 - t0) / n
    print(json.dumps({"probe": "mfma", "flops_per_launch": flops, "launches": n, "launch_us": launch_s * 1e6,
                      "tflops": flops / launch_s / 1e12, "frac_of_peak": flops / launch_s / MFMA_BF16_PEAK,
                      "power_w": p, "gfx_mhz": clk, "samples": ns, "idle_power_w": idle[0],
                      "idle_gfx_mhz": idle[1], "amd_smi": ps.ok}))


def measure_decode_append(sess, W, hq, lengths, s_q, dims, n_cached, build_s, reps=50):
    """The append of a decode step (mla_cache_append, and mla_cache_append_ws
    where it applies, of the batch's B * s_q
    newest tokens, one call; here the last s_q tokens of every sequence are
    written again from their own hidden states), timed with HIP events on
    the launch stream, median of `reps`, against its HBM bound (the 576 x
    d_model weight rows, the h rows and the written rows at 8 TB/s); and the
    cache build's rate (whole-sequence calls, wall clock) against its MFMA
    bound (2 x 576 x d_model flops a token at 2.5 PF/s).  Each timed append
    is queued behind a 512 MiB fill, so that the start event fires only when
    the append's launch is already in the queue (on an idle stream the
    interval would hold the host's launch overhead); the fill also leaves
    the weights out of the caches, as a decode step finds them."""
    import numpy as np
    import torch
    dev = hq.device
    n = hq.shape[0]
    seq_id = torch.repeat_interleave(torch.arange(len(lengths), dtype=torch.int32), s_q).to(dev)
    pos = torch.cat([torch.arange(int(Lb) - s_q, int(Lb), dtype=torch.int32) for Lb in lengths]).to(dev)
    stream = torch.cuda.current_stream()
    pad = torch.empty(1 << 27, dtype=torch.float32, device=dev)

    def timed(ws):
        for _ in range(5):
            sess.append_rows(hq, seq_id, pos, W, ws=ws)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            pad.zero_()
            e0.record(stream)
            sess.append_rows(hq, seq_id, pos, W, ws=ws)
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    t = timed(False)
    from mla_latent_kv_29_amd import _lib as L
    ws_bytes = L.mla_append_workspace_bytes(sess.cdims, sess.act, n)
    t_ws = timed(True) if ws_bytes else None
    del pad
    d = dims["d_c"] + dims["d_rope"]
    row_bytes = sess.page_bytes // dims["page_size"]
    byts = d * dims["d_model"] * 2 + n * dims["d_model"] * 2 + n * row_bytes
    t_bound = byts / HBM_PEAK
    flops_tok = 2.0 * d * dims["d_model"]
    return {"decode_tokens": n, "decode_us": t * 1e6, "decode_bound_us": t_bound * 1e6,
            "decode_frac": t_bound / t, "decode_bytes": byts,
            "decode_ws_us": t_ws * 1e6 if t_ws else None, "decode_ws_frac": t_bound / t_ws if t_ws else None,
            "ws_kernels": "k_skinny (k-group partials) + k_append_reduce (mla_cache_append_ws)" if t_ws else None,
            "kernel": ("k_append_rows" if (dims["d_c"], dims["d_rope"]) == (512, 64) and hq.dtype == torch.bfloat16
                       and dims["d_model"] % 256 == 0 and n <= 4096 else "other") + " (mla_cache_append)",
            "build_tokens_per_s": n_cached / build_s,
            "build_bound_tokens_per_s": MFMA_BF16_PEAK / flops_tok}


def run_phase_power(workload, secs, phases, stream):
    """Each phase launched back to back for `secs` seconds (in batches of 100
    launches, then a synchronisation), idle before and after; power and clock
    averaged over the samples inside each window (the first 0.3 s skipped)."""
    import torch
    ps = PowerSampler()
    time.sleep(1.0)
    res = {"probe": "phase_power", "workload": workload, "seconds": secs, "phases": []}

    def window(name, t0, t1, launch_us=None, gpu_us=None):
        p, clk, n = ps.mean(t0 + 0.3, t1)
        r = {"phase": name, "power_w": p, "gfx_mhz": clk, "samples": n}
        if launch_us is not None:
            r.update({"launch_us": launch_us, "gpu_us": gpu_us,
                      "energy_mj": p * launch_us * 1e-3 if p is not None else None})
        res["phases"].append(r)

    t0 = time.time()
    time.sleep(secs)
    window("idle", t0, time.time())
    for name, f in phases.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(20):
            f(i)
        e0.record(stream)
        for i in range(200):
            f(i)
        e1.record(stream)
        e1.synchronize()
        gpu_us = e0.elapsed_time(e1) * 1e3 / 200
        n, t0 = 0, time.time()
        while time.time() - t0 < secs:
            for i in range(100):
                f(n + i)
            n += 100
            torch.cuda.synchronize()
        t1 = time.time()
        window(name, t0, t1, (t1 - t0) * 1e6 / n, gpu_us)
    ps.stop = True
    res["amd_smi"] = ps.ok
    print(json.dumps(res))


def run_layers(args, name):
    """Layer-stack workload: one step = for every layer, mla_decode_query +
    mla_decode_attend + mla_combine + mla_output_project, each layer with its
    own paged cache (built from the same hidden states through its own W^DKV,
    W^KR) and its own weights.  Every layer takes the same seeded query rows:
    no norm, residual or MoE sits between the layers on this path, so the
    values feeding each layer are synthetic either way."""
    import numpy as np
    import torch
    from mla_latent_kv_29_amd import inputs
    from mla_latent_kv_29_amd import _lib as L
    from mla_latent_kv_29_amd.session import DecodeSession

    torch.cuda.set_device(0)
    dev = "cuda:0"
    spec = inputs.LAYER_WORKLOADS[name]
    dims, wl, n_layers = spec["dims"], spec["index"], spec["layers"]
    tdt = inputs.torch_dtype(spec["act"])
    lengths = inputs.seqlens(spec["lengths"], spec["batch"], 0, wl)
    table, pool = inputs.block_table(lengths, dims["page_size"], spec["table"], 0, wl)
    gen_h = lambda b, t0, t1: inputs.hidden(dims, b, t0, t1, tdt, dev, 0, wl)
    s_q, batch = spec["s_q"], spec["batch"]
    tau = 1.0 / math.sqrt(dims["d_head"] + dims["d_rope"])
    layers = []
    t0 = time.perf_counter()
    for li in range(n_layers):
        W = inputs.weights(dims, spec["sigma"], tdt, dev, li, wl)
        W["W_O"] = inputs.out_weight(dims, spec["sigma"], tdt, dev, li, wl)
        sess = DecodeSession(dims, spec["act"], spec["cache"], lengths, table, pool, s_q, 0, dev)
        sess.build_from_h(gen_h, W, chunk=32768)
        del W["W_DKV"], W["W_KR"]  # cache projections: not part of a decode step
        layers.append((sess, W))
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t0
    hq = torch.cat([gen_h(b, int(Lb) - s_q, int(Lb)) for b, Lb in enumerate(lengths)], 0).contiguous()
    R = batch * s_q
    y = torch.empty((R, dims["d_model"]), dtype=tdt, device=dev)
    c = layers[0][0].cdims
    act = layers[0][0].act
    owsb = L.mla_output_project_workspace_bytes(c, act, R)
    ows = torch.empty(max(owsb, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def layer(sess, W, e=None):
        dargs = (c, act, hq, batch, s_q, W["W_DQ"], W["W_UQ"], W["W_UK"], sess.cache, sess.block_table,
                 sess.max_pages, sess.seqlens, tau, sess.num_splits, sess.ws, sess.ws_bytes, sp)
        L.mla_decode_query(*dargs)
        if e is not None:
            e[0].record(stream)
        L.mla_decode_attend(*dargs)
        if e is not None:
            e[1].record(stream)
        L.mla_combine(c, act, batch, s_q, sess.num_splits, sess.ws, sess.ws_bytes, W["W_UV"], sess.out, sess.lse, sp)
        L.mla_output_project(c, act, R, sess.out, W["W_O"], y, ows, owsb, sp)

    def step(ev=None):
        for li, (sess, W) in enumerate(layers):
            layer(sess, W, None if ev is None else ev[li])

    sampled = set(range(0, args.steps, max(1, args.steps // 4)))
    evs = {i: [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in layers] for i in sampled}
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    a_ms = [e[0].elapsed_time(e[1]) for i in sampled for e in evs[i]]
    ms_per_step = wall / args.steps * 1e3
    alg = algorithmic(spec, dims, lengths)
    attn_s = float(np.mean(a_ms)) * 1e-3
    tokens = float(np.sum(lengths))
    wo_bytes = 2 * dims["d_model"] * dims["n_heads"] * dims["d_head"]
    tok_bytes = (dims["d_c"] + dims["d_rope"]) * 2
    # one layer: the decode step's bytes and flops plus W^O (weights, y rows)
    layer_bytes = alg["step_bytes"] + wo_bytes + 2 * R * dims["d_model"]
    layer_flops = alg["step_flops"] + 2 * R * dims["d_model"] * dims["n_heads"] * dims["d_head"]
    t_bound = n_layers * max(layer_bytes / HBM_PEAK, layer_flops / MFMA_BF16_PEAK)
    res = {
        "metric": f"MLA decode through {n_layers} attention layers (W^O included): cached token-layers/s",
        "value": tokens * n_layers / (ms_per_step * 1e-3),
        "unit": "cached-token-layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec["act"],
        "data": "synthetic (seeded N(0,1) hidden states, N(0,sigma^2) weights per layer at DeepSeek-V3 MLA shapes)",
        "config": {"workload": name, "batch": batch, "seq_len": spec["lengths"][1], "s_q": s_q,
                   "layers": n_layers, "cache": spec["cache"], "splits": layers[0][0].num_splits},
        "roofline": {"bound": "hbm", "achieved": alg["attn_bytes"] / attn_s / 1e9, "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": alg["attn_bytes"] / attn_s / HBM_PEAK, "traffic": None,
                     "kernel": "k_attn_v3b<false> (mla_decode_attend), every layer", "attn_ms_mean": attn_s * 1e3},
        "step_roofline": {"t_bound_us": t_bound * 1e6, "frac": t_bound / (ms_per_step * 1e-3),
                          "layer_bytes": layer_bytes, "layer_flops": layer_flops},
        "sequences_tokens_per_s": batch * s_q / (ms_per_step * 1e-3),
        "ms_per_layer": ms_per_step / n_layers,
        "cache_bytes_per_token_all_layers": n_layers * tok_bytes,
        "cache_bytes_total": int(tokens) * n_layers * tok_bytes,
        "cache_build_s": build_s,
    }
    print(json.dumps(res))


def run_fp8_proj(args, name):
    """FP8 projection workload: one step = mla_fp8_gemm for every MLA weight
    of a layer (W^O included) at the decode row count, the weights quantised
    once beforehand in 128 x 128 blocks (three copies rotated, so that no step
    finds them in the 256 MB MALL).  The W^O call, the largest, is timed with
    HIP events on its stream every step."""
    import numpy as np
    import torch
    from mla_latent_kv_29_amd import inputs
    from mla_latent_kv_29_amd import _lib as L

    torch.cuda.set_device(0)
    dev = "cuda:0"
    spec = inputs.FP8_WORKLOADS[name]
    M, wl = spec["rows"], spec["index"]
    sets = []
    for r in range(max(1, args.rotate)):
        one = []
        for pname, N, K in inputs.FP8_PROJECTIONS:
            X, W = inputs.gemm_operands(M, N, K, spec["sigma"], torch.bfloat16, dev, r, wl)
            codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
            scales = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=dev)
            L.mla_fp8_quantize_weight(W, N, K, codes, scales)
            del W
            one.append((pname, N, K, X, codes, scales, torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
        sets.append(one)
    wsb = max(L.mla_fp8_gemm_workspace_bytes(M, N, K) for _, N, K in inputs.FP8_PROJECTIONS)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(args.steps)]

    def step(i, e=None):
        for pname, N, K, X, codes, scales, Y in sets[i % len(sets)]:
            if e is not None and pname == "W_O":
                e[0].record(stream)
            L.mla_fp8_gemm(M, N, K, X, codes, scales, Y, ws, wsb, sp)
            if e is not None and pname == "W_O":
                e[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    wo_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))

    def alg_bytes(N, K):  # weight codes and scales, activations in, results out
        return N * K + (N + 127) // 128 * (K // 128) * 4 + 2 * M * K + 2 * M * N

    step_bytes = sum(alg_bytes(N, K) for _, N, K in inputs.FP8_PROJECTIONS)
    wo_bytes = alg_bytes(7168, 16384)
    achieved = wo_bytes / (wo_ms * 1e-3) / 1e9
    res = {
        "metric": f"FP8 block-scaled MLA projection GEMMs at {M} rows (E4M3, 128x128 weight blocks, 1x128 "
                  f"activation tiles): algorithmic GB/s + % HBM roofline, 1 GPU",
        "value": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 x fp8-e4m3 -> f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,sigma^2) weights at DeepSeek-V3 MLA shapes)",
        "config": {"workload": name, "rows": M, "weights": [p[0] for p in inputs.FP8_PROJECTIONS],
                   "rotation_sets": len(sets)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved * 1e9 / HBM_PEAK, "traffic": None,
                     "kernel": "mla_fp8_gemm on W^O (k_quant_x + k_skinny_f8 + k_reduce_rows)", "call_ms_mean": wo_ms},
        "step_roofline": {"t_bound_us": step_bytes / HBM_PEAK * 1e6, "frac": step_bytes / HBM_PEAK / (ms_per_step * 1e-3),
                          "step_bytes": step_bytes},
    }
    print(json.dumps(res))


def run_prefill(args, name):
    """Prefill workload: one step = mla_prefill_project + mla_prefill_attend
    over the packed sequences; the attention (the dominant kernel) is timed
    with HIP events around its call on its stream, every step."""
    import numpy as np
    import torch
    from mla_latent_kv_29_amd import inputs
    from mla_latent_kv_29_amd import _lib as L

    torch.cuda.set_device(0)
    dev = "cuda:0"
    spec = inputs.PREFILL_WORKLOADS[name]
    dims, wl = spec["dims"], spec["index"]
    tdt = inputs.torch_dtype(spec["act"])
    lengths = inputs.seqlens(spec["lengths"], spec["batch"], 0, wl)
    W = inputs.weights(dims, spec["sigma"], tdt, dev, 0, wl)
    h = torch.cat([inputs.hidden(dims, b, 0, int(Lb), tdt, dev, 0, wl) for b, Lb in enumerate(lengths)], 0)
    h = h.contiguous()
    n = int(h.shape[0])
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=dev)
    c = L.make_dims(dims)
    wsb = L.mla_prefill_workspace_bytes(c, L.MLA_BF16, n)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    out = torch.empty((n, dims["n_heads"], dims["d_head"]), dtype=tdt, device=dev)
    lse = torch.empty((n, dims["n_heads"]), dtype=torch.float32, device=dev)
    tau = 1.0 / math.sqrt(dims["d_head"] + dims["d_rope"])
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    pargs = (c, L.MLA_BF16, h, n, len(lengths), cu, int(max(lengths)), W["W_DQ"], W["W_UQ"], W["W_UK"], W["W_UV"],
             W["W_DKV"], W["W_KR"], tau, out, lse, ws, wsb, sp)
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]

    def step(e=None):
        if e is not None:
            e[0].record(stream)
        L.mla_prefill_project(*pargs)
        if e is not None:
            e[1].record(stream)
        L.mla_prefill_attend(*pargs)
        if e is not None:
            e[2].record(stream)

    if args.phase_power > 0:
        step()
        torch.cuda.synchronize()
        phases = {"step": lambda i: step(), "project": lambda i: L.mla_prefill_project(*pargs),
                  "attend": lambda i: L.mla_prefill_attend(*pargs)}
        run_phase_power(name, args.phase_power, phases, stream)
        return

    copy_calibration(args.copy_calibration, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    p_ms = [e[0].elapsed_time(e[1]) for e in ev]
    a_ms = [e[1].elapsed_time(e[2]) for e in ev]
    ms_per_step = wall / args.steps * 1e3
    attn_flops, proj_flops = prefill_algorithmic(dims, lengths)
    attn_s = float(np.mean(a_ms)) * 1e-3
    achieved = attn_flops / attn_s / 1e12
    t_bound = (attn_flops + proj_flops) / MFMA_BF16_PEAK
    res = {
        "metric": f"MLA prefill tokens/s + % MFMA roofline, {spec['batch']} x {spec['lengths'][1]} tokens bf16, 1 GPU",
        "value": n / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec["act"],
        "data": "synthetic (seeded N(0,1) hidden states, N(0,sigma^2) weights at DeepSeek-V3 MLA shapes)",
        "config": {"workload": name, "batch": int(spec["batch"]), "seq_len": int(spec["lengths"][1]),
                   "tokens": n},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
                     "frac": achieved * 1e12 / MFMA_BF16_PEAK, "traffic": measured_traffic(name, "prefill"),
                     "kernel": "k_prefill_attn (mla_prefill_attend)", "attn_ms_mean": float(np.mean(a_ms)),
                     "attn_flops": attn_flops},
        "step_roofline": {"t_bound_us": t_bound * 1e6, "frac": t_bound / (ms_per_step * 1e-3),
                          "step_flops": attn_flops + proj_flops},
        "phases_ms": {"project": float(np.median(p_ms)), "attend": float(np.median(a_ms))},
    }
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="v3_bf16_b64_l4096")
    ap.add_argument("--splits", type=int, default=0, help="KV splits per sequence (0 = library default)")
    ap.add_argument("--rotate", type=int, default=3, help="copies of cache+weights rotated across steps")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="measure achievable HBM read and copy bandwidth (75 MB, 302 MB) and exit")
    ap.add_argument("--phase-power", type=float, default=0.0, metavar="SECS",
                    help="run idle, the whole step, and each phase (decode: attention, query, combine; "
                         "prefill: projections, attention) back to back "
                         "for SECS seconds each while amd-smi samples board power and clocks; print one "
                         "JSON line of per-phase launch time, power, clock and energy per launch, and exit")
    ap.add_argument("--mfma-probe", type=float, default=0.0, metavar="SECS",
                    help="run the register-only bf16 MFMA probe back to back for SECS seconds while amd-smi "
                         "samples power and clocks; print one JSON line of the achieved MFMA rate and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain elementwise copy of MIB MiB three times (untimed), as the "
                         "reference for hardware byte counters")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="store the attention's HBM bytes of --workload from two rocprofv3 counter files "
                         "(FETCH_SIZE, WRITE_SIZE) in profiles/attn_traffic.json; no GPU work")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build measures one GPU's "
              f"share at its real shape and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    if args.mfma_probe > 0:
        run_mfma_probe(args.mfma_probe)
        return
    if args.hbm_probe:
        run_hbm_probe(args)
        return
    from mla_latent_kv_29_amd import inputs
    if args.workload in inputs.PREFILL_WORKLOADS:
        run_prefill(args, args.workload)
        return
    if args.workload in inputs.LAYER_WORKLOADS:
        run_layers(args, args.workload)
        return
    if args.workload in inputs.FP8_WORKLOADS:
        run_fp8_proj(args, args.workload)
        return

    import numpy as np
    import torch
    from mla_latent_kv_29_amd import _lib as L
    from mla_latent_kv_29_amd.session import DecodeSession

    torch.cuda.set_device(0)
    dev = "cuda:0"
    spec = inputs.WORKLOADS[args.workload]
    dims = spec["dims"]
    wl = spec["index"]
    tdt = inputs.torch_dtype(spec["act"])
    lengths = inputs.seqlens(spec["lengths"], spec["batch"], 0, wl)
    table, pool = inputs.block_table(lengths, dims["page_size"], spec["table"], 0, wl)
    W = inputs.weights(dims, spec["sigma"], tdt, dev, 0, wl)
    sess = DecodeSession(dims, spec["act"], spec["cache"], lengths, table, pool, spec["s_q"], args.splits, dev)
    gen_h = lambda b, t0, t1: inputs.hidden(dims, b, t0, t1, tdt, dev, 0, wl)

    # ---- cache build (not part of the step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sess.build_from_h(gen_h, W, chunk=32768)
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t0
    s_q = spec["s_q"]
    hq = torch.cat([gen_h(b, int(Lb) - s_q, int(Lb)) for b, Lb in enumerate(lengths)], 0).contiguous()
    tau = 1.0 / math.sqrt(dims["d_head"] + dims["d_rope"])
    append = measure_decode_append(sess, W, hq, lengths, s_q, dims, int(sum(int(x) for x in lengths)), build_s)

    # ---- rotation sets: same values in distinct buffers
    sets = [(sess.pages, W)]
    for _ in range(1, max(1, args.rotate)):
        sets.append((sess.pages.clone(), {k: v.clone() for k, v in W.items()}))
    caches = [L.cache_struct(p, sess.cache_dtype, sess.num_pages) for p, _ in sets]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    c = sess.cdims
    dargs = lambda i: (c, sess.act, hq, sess.batch, s_q, sets[i][1]["W_DQ"], sets[i][1]["W_UQ"], sets[i][1]["W_UK"],
                       caches[i], sess.block_table, sess.max_pages, sess.seqlens, tau, sess.num_splits, sess.ws,
                       sess.ws_bytes, sp)
    every = max(1, args.steps // 64)  # timed steps whose phases the events bracket
    sampled = list(range(0, args.steps, every))
    ev = {i: tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for i in sampled}

    fp8w = spec.get("weights") == "fp8"
    if fp8w:
        # E4M3 weights with 128 x 128-block scales, quantised by the library once per rotation set
        qsets = [sess.quantize_fp8w(Wk) for _, Wk in sets]
        sess.fp8w_workspace()
        fargs = lambda i: (c, hq, sess.batch, s_q, qsets[i]["W_DQ"], qsets[i]["W_UQ"], qsets[i]["W_UKT"], caches[i],
                           sess.block_table, sess.max_pages, sess.seqlens, tau, sess.num_splits, sess.ws,
                           sess.ws_bytes, sp)

    def query(k):
        if fp8w:
            L.mla_decode_fp8w_query(*fargs(k))
        else:
            L.mla_decode_query(*dargs(k))

    def attend(k):
        L.mla_decode_attend(*dargs(k))

    def combine(k):
        if fp8w:
            L.mla_combine_fp8w(c, sess.batch, s_q, sess.num_splits, sess.ws, sess.ws_bytes, qsets[k]["W_UV"],
                               sess.out, sess.lse, sp)
        else:
            L.mla_combine(c, sess.act, sess.batch, s_q, sess.num_splits, sess.ws, sess.ws_bytes,
                          sets[k][1]["W_UV"], sess.out, sess.lse, sp)

    def step(i, e=None):
        k = i % len(sets)
        if e is not None:
            e[0].record(stream)
        query(k)
        if e is not None:
            e[1].record(stream)
        attend(k)
        if e is not None:
            e[2].record(stream)
        combine(k)
        if e is not None:
            e[3].record(stream)

    if args.phase_power > 0:
        step(0)
        torch.cuda.synchronize()
        phases = {"step": lambda i: step(i), "attend": lambda i: attend(i % len(sets)),
                  "query": lambda i: query(i % len(sets)), "combine": lambda i: combine(i % len(sets))}
        run_phase_power(args.workload, args.phase_power, phases, stream)
        return

    copy_calibration(args.copy_calibration, dev)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, ev.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    q_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in sampled]
    a_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in sampled]
    c_ms = [ev[i][2].elapsed_time(ev[i][3]) for i in sampled]
    s_ms = [ev[i][0].elapsed_time(ev[i][3]) for i in sampled]
    ms_per_step = wall / args.steps * 1e3
    tokens = float(np.sum(lengths))
    alg = algorithmic(spec, dims, lengths)

    attn_s = float(np.mean(a_ms)) * 1e-3
    # the attention's roof is the larger of its byte time and its MFMA time
    # (bf16 at one query row: bytes; fp8 or several query rows: MFMA)
    if alg["attn_flops"] / MFMA_BF16_PEAK > alg["attn_bytes"] / HBM_PEAK:
        bound, achieved, peak, unit = "mfma", alg["attn_flops"] / attn_s / 1e12, MFMA_BF16_PEAK / 1e12, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", alg["attn_bytes"] / attn_s / 1e9, HBM_PEAK / 1e9, "GB/s"
    t_bound = max(alg["step_bytes"] / HBM_PEAK, alg["step_flops"] / MFMA_BF16_PEAK)
    res = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "cached-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "bf16+fp8cache", "fp8e8": "bf16+fp8cache(ue8m0 scales)"}.get(spec["cache"], spec["act"])
                 + ("+fp8weights" if fp8w else ""),
        "data": "synthetic (seeded N(0,1) hidden states, N(0,sigma^2) weights at DeepSeek-V3 MLA shapes)",
        "config": {"workload": args.workload, "batch": int(spec["batch"]), "seq_len": spec["lengths"][1]
                   if spec["lengths"][0] == "fixed" else f"U[{spec['lengths'][1]},{spec['lengths'][2]}]",
                   "s_q": s_q, "cache": spec["cache"], "weights": spec.get("weights", spec["act"]),
                   "splits": sess.num_splits,
                   "cached_tokens": int(tokens), "rotation_sets": len(sets)},
        "roofline": {"scope": "dominant kernel (the split-KV attention launch) only; the whole step is in "
                              "step_roofline",
                     "bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
                     "traffic": measured_traffic(args.workload, spec["cache"], sess.num_splits),
                     "kernel": {"bf16": "k_attn_v3b<false>", "fp8": "k_attn_v3b<true>", "fp8e8": "k_attn_v3b<true, true>"}[spec["cache"]]
                     + " (mla_decode_attend)",
                     "attn_ms_mean": float(np.mean(a_ms))},
        "step_roofline": {"t_bound_us": t_bound * 1e6, "frac": t_bound / (ms_per_step * 1e-3),
                          "step_bytes": alg["step_bytes"], "step_flops": alg["step_flops"]},
        "phases_ms": {"query": float(np.median(q_ms)), "attend": float(np.median(a_ms)),
                      "combine": float(np.median(c_ms))},
        # per-step times of the sampled steps (events at both ends of each, so
        # each includes one event's wait): p10 / p50 / p90, and the mean
        "step_ms_sampled": {"p10": float(np.percentile(s_ms, 10)), "p50": float(np.percentile(s_ms, 50)),
                            "p90": float(np.percentile(s_ms, 90)), "mean": float(np.mean(s_ms)), "n": len(s_ms)},
        "cache_build_s": build_s,
        "append": append,
    }
    if s_q > 1:
        # the verify step checks s_q - 1 drafts; expected emitted tokens at the
        # pages' 85% acceptance
        tps = L.mla_mtp_tokens_per_step(MTP_ACCEPTANCE, s_q - 1)
        res["mtp_verify"] = {"depth": s_q - 1, "acceptance": MTP_ACCEPTANCE, "tokens_per_step": tps,
                             "generated_tokens_per_s": spec["batch"] * tps / (ms_per_step * 1e-3)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, dims, W, gen_h, lengths, args.cpu_budget)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
