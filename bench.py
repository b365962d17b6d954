"""Benchmark of the KIVI KV-cache codec on one MI355X.

One step = the whole full-cache hot path over one synthetic cache: per-channel
key encode, per-token value encode, key decode, value decode, each as one
call over every (layer, batch, head) slice, with the residual window of R
recent tokens left in fp16.  Inputs are generated on the GPU before timing.

Prints one JSON line.  ``value`` is the fp16-equivalent encode+decode
throughput: (fp16 bytes of K and V consumed by encode + produced by decode)
per second.  ``roofline`` is for the kernel with the largest share of the
step, from HIP events on the stream the kernels run on; ``cpu_baseline`` is
the numpy oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E, 8 TB/s


def algorithmic_bytes(kind: str, direction: str, S: int, n: int, D: int, G: int, b: int) -> int:
    """Bytes one launch must move: fp16 data plus packed codes plus fp16 sidecars
    (padding slots included, since they are written/read)."""
    fp16 = S * n * D * 2
    if kind == "k":
        ng = -(-n // G)
        codes = S * ng * (G * b // 32) * D * 4
        stats = 2 * S * ng * D * 2
    else:
        ngv = -(-D // G)
        codes = S * n * ngv * (G * b // 32) * 4
        stats = 2 * S * n * ngv * 2
    return fp16 + codes + stats


def attention_bytes(S: int, n: int, R: int, D: int, G: int, kb: int, vb: int, r: int,
                    n_splits: int) -> dict:
    """Bytes of one decode-attention call.  ``method``: what the attention
    itself must move -- the packed prefix (codes + sidecars, padding slots of
    partial key groups included), the fp16 residual, q and the output.
    ``partials``: the split plan's partial sums, written by the attention
    kernel and read back by the merge kernel (0 with one split), an artefact
    of this implementation reported on its own."""
    ngk, ngv = -(-n // G), -(-D // G)
    payload = (S * ngk * (G * kb // 32) * D * 4 + 2 * S * ngk * D * 2
               + S * n * ngv * (G * vb // 32) * 4 + 2 * S * n * ngv * 2)
    resid = 2 * S * R * D * 2
    q = out = S * r * D * 2
    partials = 2 * S * n_splits * r * (D + 2) * 4 if n_splits > 1 else 0
    return {"method": payload + resid + q + out, "partials": partials}


def kernel_source_hash() -> str:
    path = os.path.join(ROOT, "kv_cache_quantization_codec_amd", "csrc", "kivi_kernels.hip")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of ``kernel`` measured with rocprofv3 counters and
    scaled by a copy of known size (profiles/traffic_<workload>.txt), or None
    when no such record exists or it was taken on another kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            key, val = (x.strip() for x in line.split("=", 1))
            rec[key] = val
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return int(rec[kernel]) if kernel in rec else None


CODEC_KERNELS = ("encode_k", "encode_v", "decode_k", "decode_v")


def _codec_kernel(name: str):
    """Which codec kernel a rocprofv3 kernel name is, or None (value encode
    at G = 32 launches encode_v_quad_kernel)."""
    for k in CODEC_KERNELS:
        for form in (f"{k}_kernel<", f"{k}_quad_kernel<"):
            if f"kivi::(anonymous namespace)::{form}" in name:
                return k
    return None


def summarize_traffic(workload: str, fetch_csv: str, write_csv: str) -> str:
    """Text of profiles/traffic_<workload>.txt from two rocprofv3 --pmc runs of
    this script (FETCH_SIZE, then WRITE_SIZE; counter_collection CSVs).

    Calibration: the set-up assembles the cache with 2 * layers device
    copies of one layer's K or V (slices_per_layer * tokens * head_dim fp16,
    known size); they are the widest-grid dispatches of the runtime's copy
    kernel before the first codec kernel.  Each counter is scaled by known
    bytes / counted KiB on those copies."""
    import csv

    from kvsynth import WORKLOADS
    w = WORKLOADS[workload]
    copy_bytes = w.slices_per_layer * w.tokens * w.head_dim * 2
    n_copies = 2 * w.layers

    def read(path, counter):
        setup, per = [], {k: [] for k in CODEC_KERNELS}
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            val = float(r["Counter_Value"])
            kern = _codec_kernel(r["Kernel_Name"])
            if kern:
                per[kern].append(val)
            elif r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer") and not any(per.values()):
                setup.append((int(r["Grid_Size"]), val))
        widest = max((g for g, _ in setup), default=0)
        copies = [v for g, v in setup if g == widest]
        if len(copies) != n_copies or not all(per.values()):
            raise SystemExit(f"{path}: expected {n_copies} set-up copies and every codec kernel, "
                             f"found {len(copies)} copies")
        scale = copy_bytes / (sum(copies) / len(copies) * 1024.0)
        return scale, {k: sum(v) / len(v) for k, v in per.items()}

    fs, fetch = read(fetch_csv, "FETCH_SIZE")
    ws, write = read(write_csv, "WRITE_SIZE")
    # the profiler's output directories, as given on the command line
    fetch_dir = os.path.dirname(os.path.relpath(fetch_csv, ROOT))
    write_dir = os.path.dirname(os.path.relpath(write_csv, ROOT))
    fetch_csv = os.path.relpath(fetch_csv, ROOT)
    write_csv = os.path.relpath(write_csv, ROOT)
    lines = [
        "# HBM traffic per launch from rocprofv3 counters (FETCH_SIZE, WRITE_SIZE; KiB per",
        f"# dispatch, one --pmc pass each) for workload {workload}, each counter scaled by",
        f"# what it reads on the {n_copies} set-up copies of {copy_bytes} bytes each way in the",
        "# same run.  Commands, from the repository root:",
        f"#   rocprofv3 --pmc FETCH_SIZE -d {fetch_dir} -o run --output-format csv -- \\",
        f"#       python -u bench.py --workload {workload} --steps 2 --warmup 1 --no-cpu-baseline",
        f"#   rocprofv3 --pmc WRITE_SIZE -d {write_dir} -o run --output-format csv -- \\",
        f"#       python -u bench.py --workload {workload} --steps 2 --warmup 1 --no-cpu-baseline",
        f"#   python bench.py --workload {workload} --summarize-traffic \\",
        f"#       {fetch_csv} \\",
        f"#       {write_csv}",
        "# bench.py reports these bytes only while kivi_kernels.hip hashes to the value below.",
        f"kernel_source_sha256_16 = {kernel_source_hash()}",
        f"fetch_scale = {fs:.4f}",
        f"write_scale = {ws:.4f}",
    ]
    n = w.tokens - w.residual_length
    for k in CODEC_KERNELS:
        b = w.k_bits if k.endswith("k") else w.v_bits
        alg = algorithmic_bytes(k[-1], k[:6], w.slices, n, w.head_dim, w.group_size, b)
        fb, wb = fetch[k] * 1024.0 * fs, write[k] * 1024.0 * ws
        lines.append(f"# {k}: fetch {fetch[k]:.0f} KiB raw -> {fb:.0f} B, write {write[k]:.0f} KiB "
                     f"raw -> {wb:.0f} B, sum / algorithmic = {(fb + wb) / alg:.5f}")
        lines.append(f"{k} = {fb + wb:.0f}")
    return "\n".join(lines) + "\n"


def attention_bench(w, cfg, k, v, kq, vq, n, args, dev, cpu=True):
    """Decode attention of one query token per query head over the cache
    just encoded (quantized prefix + the R fp16 tokens left in k/v), all
    slices in one call; HIP events on the launch stream."""
    import torch

    import kv_cache_quantization_codec_amd as K
    from kvsynth import decode_queries

    S, D, G, r = w.slices, w.head_dim, w.group_size, w.q_per_kv
    R = w.tokens - n
    q = decode_queries(w, dev)
    out = torch.empty_like(q)
    cache = K.AttnCache(cfg, kq, vq, n, k[:, n:], v[:, n:], 0, R)
    ws_bytes = K.kivi_attention_workspace_bytes(cfg, S, r, n, R)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    sm_scale = D ** -0.5

    def call():
        K.kivi_decode_attention(cfg, cache, q, sm_scale, out, ws)

    # The first calls after the codec steps run 10-15% slow (measured: 0.85-0.88
    # ms per call over the first 20 on the Llama-2-7B shape, 0.74-0.77 ms
    # after), so warm up with as many calls as one timed run, then report the
    # median over three timed runs of back-to-back calls.
    reps = max(10, args.steps)
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    runs = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) / reps)
    ms = sorted(runs)[1]
    n_splits = ws_bytes // (S * r * (D + 2) * 4) if ws_bytes else 1
    alg = attention_bytes(S, n, R, D, G, w.k_bits, w.v_bits, r, n_splits)
    gbps = alg["method"] / (ms / 1000.0) / 1e9
    res = {
        "what": "softmax attention of one query token per query head over the packed prefix "
                "plus the fp16 residual, all layers' slices in one call",
        "q_per_kv": r,
        "cached_tokens": w.tokens,
        "n_splits": n_splits,
        "ms": round(ms, 4),
        "ms_runs": [round(x, 4) for x in runs],
        "algorithmic_bytes": alg["method"],
        "partial_sum_bytes": alg["partials"],
        "achieved_GBps": round(gbps, 1),
        "roofline_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "with_partials_GBps": round((alg["method"] + alg["partials"]) / (ms / 1000.0) / 1e9, 1),
        "fp16_cache_equiv_GBps": round(2 * S * w.tokens * D * 2 / (ms / 1000.0) / 1e9, 1),
        "decode_steps_per_s": round(1000.0 / ms, 1),
    }
    if cpu:
        res["cpu_baseline"] = attention_cpu_baseline(w, k, v, kq, vq, q, n, sm_scale, alg,
                                                     min(args.cpu_budget, 6.0))
    return res


def attention_cpu_baseline(w, k, v, kq, vq, q, n, sm_scale, alg, budget_s):
    """The float64 attention oracle, single-threaded, on whole slices of the
    same cache until about ``budget_s`` seconds; scaled to algorithmic GB/s."""
    import numpy as np

    from oracle import attention_ref as att

    S = w.slices
    done, spent, chunk = 0, 0.0, 4
    while spent < budget_s and done < S:
        sl = slice(done, min(done + chunk, S))
        kp = tuple(t[sl].cpu().numpy() for t in kq)
        vp = tuple(t[sl].cpu().numpy() for t in vq)
        qh, rk, rv = q[sl].cpu().numpy(), k[sl, n:].cpu().numpy(), v[sl, n:].cpu().numpy()
        t0 = time.perf_counter()
        att.decode_attention(qh, kp, vp, n, rk, rv, w.k_bits, w.v_bits, w.group_size, sm_scale)
        spent += time.perf_counter() - t0
        done = sl.stop
    per_slice = alg["method"] / S
    return {
        "value": round(per_slice * done / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} of {S} slices, float64 numpy attention oracle, {spent:.1f} s single-threaded",
    }


def _oracle_round_trip(kh, vh, w, cfg, n, kb, vb):
    """The numpy oracle's encode + decode of one chunk's K and V."""
    from oracle import fp8_ref as f8
    from oracle import kivi_ref as ref

    G = cfg.group_size
    if w.fp8_keys:
        f8.decode(f8.encode_keys(kh, n))
    else:
        kc, ks, kz = ref.encode_k(kh, n, kb, G)
        ref.decode_k(kc, ks, kz, n, kb, G)
    vc, vs, vz = ref.encode_v(vh, n, vb, G)
    ref.decode_v(vc, vs, vz, n, vb, G, cfg.head_dim)


def _oracle_chunks(k, v, w, cfg, chunk=8):
    """Chunks of ``chunk`` slices taken from the layers in turn, with each
    layer's bits (the oracle's boundary rule for a per-layer mix): yields
    (slice range, k_bits, v_bits)."""
    from oracle import layer_mix_ref as mix

    spl = w.slices_per_layer
    bits = mix.layer_bits(w.layers, w.boundary, (cfg.k_bits, cfg.v_bits), w.boundary_bits)
    c = 0
    while True:
        layer, off = c % w.layers, (c // w.layers) * chunk
        c += 1
        if off >= spl:
            return
        yield slice(layer * spl + off, layer * spl + min(off + chunk, spl)), bits[layer][0], bits[layer][1]


def cpu_baseline(k, v, w, cfg, n, budget_s=12.0):
    """Time the numpy oracle (single thread) on whole slices of the same cache
    until about ``budget_s`` seconds of CPU work; scale to fp16-eq GB/s.
    Chunks of 8 slices are taken from the layers in turn, each coded with
    its layer's bits."""
    done, spent, chunk = 0, 0.0, 8
    S = k.shape[0]
    for sl, kb, vb in _oracle_chunks(k, v, w, cfg, chunk):
        if spent >= budget_s:
            break
        kh = k[sl].cpu().numpy()
        vh = v[sl].cpu().numpy()
        t0 = time.perf_counter()
        _oracle_round_trip(kh, vh, w, cfg, n, kb, vb)
        spent += time.perf_counter() - t0
        done += sl.stop - sl.start
    fp16_bytes = 2 * 2 * done * n * cfg.head_dim * 2
    return {
        "value": round(fp16_bytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} of {S} slices, {chunk} at a time from the layers in turn "
                  f"({done * n} tokens x {cfg.head_dim} channels, K and V), "
                  f"numpy oracle encode+decode, {spent:.1f} s single-threaded "
                  f"(host has {len(os.sched_getaffinity(0))} cores available)",
    }


def cpu_baseline_threads(k, v, w, cfg, n, budget_s=12.0):
    """The same oracle on the same kind of sample with one thread per
    available core (numpy runs its array loops without the GIL): batches of
    chunks are copied to the host, then coded in parallel; only the coding
    is timed, until about ``budget_s`` seconds of wall-clock."""
    from concurrent.futures import ThreadPoolExecutor

    threads = len(os.sched_getaffinity(0))
    chunk = 8
    S = k.shape[0]
    chunks = _oracle_chunks(k, v, w, cfg, chunk)
    done, spent = 0, 0.0
    with ThreadPoolExecutor(threads) as pool:
        while spent < budget_s:
            batch = []
            for sl, kb, vb in chunks:
                batch.append((k[sl].cpu().numpy(), v[sl].cpu().numpy(), kb, vb))
                if len(batch) == 2 * threads:
                    break
            if not batch:
                break
            t0 = time.perf_counter()
            list(pool.map(lambda a: _oracle_round_trip(a[0], a[1], w, cfg, n, a[2], a[3]), batch))
            spent += time.perf_counter() - t0
            done += sum(a[0].shape[0] for a in batch)
    fp16_bytes = 2 * 2 * done * n * cfg.head_dim * 2
    return {
        "value": round(fp16_bytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {S} slices in chunks of {chunk} on {threads} threads, numpy oracle "
                  f"encode+decode, {spent:.1f} s wall-clock",
    }


def copy_ceiling(dev, nbytes=1 << 32, reps=10):
    """Read+write GB/s of torch's device copy kernel over ``nbytes``: the
    practical streaming ceiling, and the calibration kernel for HBM counters."""
    import torch

    src = torch.empty(nbytes // 2, dtype=torch.float16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return round(2 * nbytes / (ms / 1000.0) / 1e9, 1)


def stream_bench(w, args):
    """Streaming decode: prefill, then w.steps calls of kivi_append_flush (one
    launch each, all slices of all layers); per-step GPU time from HIP events
    on the launch stream."""
    import numpy as np
    import torch

    import kv_cache_quantization_codec_amd as K
    from kvsynth import layer_kv, stream_tokens

    cfg = K.Config(w.k_bits, w.v_bits, w.group_size, w.residual_length, w.head_dim)
    S, T, D, G = w.slices, w.tokens, w.head_dim, w.group_size
    dev = torch.device("cuda:0")
    k = torch.empty((S, T, D), dtype=torch.float16, device=dev)
    v = torch.empty_like(k)
    spl = w.slices_per_layer
    for layer in range(w.layers):
        kl, vl = layer_kv(w, layer, device=dev)
        k[layer * spl:(layer + 1) * spl] = kl
        v[layer * spl:(layer + 1) * spl] = vl
        del kl, vl
    kn, vn = stream_tokens(w, w.steps, device=dev)
    cap = -(-(T + w.steps) // G) * G

    def run(record):
        st = K.Stream(cfg, S, cap, dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        K.kivi_stream_prefill(st, k, v, T)
        e1.record()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(w.steps + 1)]
        flushed = []
        ev[0].record()
        for i in range(w.steps):
            flushed.append(K.kivi_append_flush(st, kn[i], vn[i]))
            ev[i + 1].record()
        torch.cuda.synchronize()
        step_us = [ev[i].elapsed_time(ev[i + 1]) * 1000.0 for i in range(w.steps)]
        return e0.elapsed_time(e1), step_us, flushed, st

    for _ in range(max(args.warmup, 1)):
        run(False)
    t0 = time.perf_counter()
    prefill_ms, step_us, flushed, st = run(True)
    wall = time.perf_counter() - t0
    fl = np.array([u for u, f in zip(step_us, flushed) if f])
    nf = np.array([u for u, f in zip(step_us, flushed) if not f])
    allv = np.array(step_us)
    nq = (T - w.residual_length) // G * G
    prefill_bytes = (algorithmic_bytes("k", "encode", S, nq, D, G, w.k_bits)
                     + algorithmic_bytes("v", "encode", S, nq, D, G, w.v_bits)
                     + 2 * S * (T - nq) * D * 2 * 2)
    # every step: read k_new and v_new, write both into the rings, and write
    # the new value row's codes and sidecars (values are quantized on arrival);
    # a flush step also encodes one key group (read G ring rows, write codes)
    ngv = -(-D // G)
    append_bytes = (2 * 2 * S * D * 2
                    + S * (ngv * (G * w.v_bits // 32) * 4 + 2 * ngv * 2))
    flush_bytes = algorithmic_bytes("k", "encode", S, G, D, G, w.k_bits)
    pct = lambda a, q: round(float(np.percentile(a, q)), 2) if len(a) else None
    offload = offload_bench(w, cfg, st, cap, dev)
    return {
        "metric": "streaming decode step latency (append 1 token per slice; flush a group "
                  "when the fp16 residual exceeds R), 1 MI355X",
        "value": pct(allv, 50),
        "unit": "us",
        "n_gpus": 1,
        "steps": w.steps,
        "warmup": max(args.warmup, 1),
        "ms_per_step": round(float(allv.mean()) / 1000.0, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "batch": w.batch, "kv_heads": w.heads,
                   "head_dim": D, "prefill_tokens": T, "k_bits": w.k_bits, "v_bits": w.v_bits,
                   "group_size": G, "residual_length": w.residual_length},
        "p99_us": pct(allv, 99),
        "flush_steps": int(len(fl)),
        "flush_p50_us": pct(fl, 50), "flush_p99_us": pct(fl, 99),
        "append_p50_us": pct(nf, 50), "append_p99_us": pct(nf, 99),
        "append_GBps": round(append_bytes / (float(np.median(nf)) * 1e-6) / 1e9, 1) if len(nf) else None,
        "flush_GBps": round((append_bytes + flush_bytes) / (float(np.median(fl)) * 1e-6) / 1e9, 1)
        if len(fl) else None,
        "prefill_ms": round(prefill_ms, 3),
        "prefill_GBps": round(prefill_bytes / (prefill_ms * 1e-3) / 1e9, 1),
        "host_wall_steps_per_s": round(w.steps / wall, 1),
        "final_state": {"n_quant": st.n_quant, "residual": st.ring_count},
        "offload_restore": offload,
    }


def offload_bench(w, cfg, st, cap, dev):
    """Compact host image of the streaming cache after the decode steps:
    device-to-host offload and host-to-device restore (into a second stream)
    through pinned memory, timed with HIP events, against a plain fp16 copy
    of the same tokens' size class over the same link."""
    import torch

    import kv_cache_quantization_codec_amd as K

    S, D = w.slices, w.head_dim
    nbytes = K.kivi_stream_image_bytes(cfg, S, st.n_quant)
    host = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    dst = K.Stream(cfg, S, cap, dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    off_ms = timed(lambda: K.kivi_stream_offload(st, host))
    res_ms = timed(lambda: K.kivi_stream_restore(dst, host, st.n_quant, st.ring_head, st.ring_count))
    # the same link moving fp16: a 2 GiB device -> pinned host copy, and back
    probe = torch.empty(1 << 30, dtype=torch.float16, device=dev)
    hprobe = torch.empty(1 << 30, dtype=torch.float16).pin_memory()
    d2h_ms = timed(lambda: hprobe.copy_(probe, non_blocking=True))
    h2d_ms = timed(lambda: probe.copy_(hprobe, non_blocking=True))
    tokens = st.n_quant + st.ring_count
    fp16_bytes = 2 * S * tokens * D * 2
    d2h_gbps = probe.numel() * 2 / (d2h_ms * 1e-3) / 1e9
    h2d_gbps = probe.numel() * 2 / (h2d_ms * 1e-3) / 1e9
    return {
        "what": "host image of the whole streaming cache (quantized prefix + fp16 residual ring) "
                "through pinned memory; restore includes re-quantizing the residual value rows",
        "cached_tokens": tokens,
        "image_bytes": nbytes,
        "fp16_bytes": fp16_bytes,
        "compression": round(fp16_bytes / nbytes, 3),
        "offload_ms": round(off_ms, 3),
        "restore_ms": round(res_ms, 3),
        "offload_link_GBps": round(nbytes / (off_ms * 1e-3) / 1e9, 2),
        "restore_link_GBps": round(nbytes / (res_ms * 1e-3) / 1e9, 2),
        "offload_fp16_equiv_GBps": round(fp16_bytes / (off_ms * 1e-3) / 1e9, 2),
        "restore_fp16_equiv_GBps": round(fp16_bytes / (res_ms * 1e-3) / 1e9, 2),
        "fp16_copy_d2h_GBps": round(d2h_gbps, 2),
        "fp16_copy_h2d_GBps": round(h2d_gbps, 2),
    }


def _median(xs):
    return float(statistics.median(xs))


def build_cache(w, dev):
    """The workload's K and V of all layers, [L*B*H, T, D] fp16 each, generated
    on the device one layer at a time."""
    import torch

    from kvsynth import layer_kv

    k = torch.empty((w.slices, w.tokens, w.head_dim), dtype=torch.float16, device=dev)
    v = torch.empty_like(k)
    spl = w.slices_per_layer
    for layer in range(w.layers):
        kl, vl = layer_kv(w, layer, device=dev)
        k[layer * spl:(layer + 1) * spl] = kl
        v[layer * spl:(layer + 1) * spl] = vl
        del kl, vl
    return k, v


def time_steps(calls, steps, warmup):
    """Runs ``warmup`` untimed steps, then ``steps`` timed steps of the calls
    in order, with a HIP event (on torch's current stream, where the binding
    launches) before and after every call.  Returns (wall ms per step,
    per-call ms lists, per-step ms list)."""
    import torch

    torch.cuda.synchronize()
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        for j, c in enumerate(calls):
            c()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per_call = [[ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)] for j in range(len(calls))]
    per_step = [ev[i][0].elapsed_time(ev[i][len(calls)]) for i in range(steps)]
    return (t1 - t0) * 1000.0 / steps, per_call, per_step


def codec_bench(w, args, dev, *, attention: bool, cpu: bool, per_layer: bool = False,
                steps: int | None = None):
    """One workload's full-cache step (encode K, encode V, decode K, decode V
    over every slice), its roofline figures, and optionally decode attention
    over the same cache, the oracle timed beside it, and the same step as a
    loop of one call per layer.  Returns the result dict; the device tensors
    are released on return."""
    import torch

    import kv_cache_quantization_codec_amd as K

    steps = args.steps if steps is None else steps
    cfg = K.Config(w.k_bits, w.v_bits, w.group_size, w.residual_length, w.head_dim)
    S, T, D, G = w.slices, w.tokens, w.head_dim, w.group_size
    n = T - w.residual_length
    k, v = build_cache(w, dev)
    ko = torch.empty((S, n, D), dtype=torch.float16, device=dev)
    vo = torch.empty_like(ko)
    names = ["encode_k", "encode_v", "decode_k", "decode_v"]
    launches = {nm: 1 for nm in names}
    spl = w.slices_per_layer
    kq = vq = None
    if w.boundary:
        # per-layer bit mix: the library's boundary rule, one config per layer,
        # each run of equal layers in one allocation (one launch per run)
        prot = set(K.kivi_boundary_layers(w.layers, w.boundary))
        cfgs = [K.Config(*(w.boundary_bits if l in prot else (w.k_bits, w.v_bits)), G,
                         w.residual_length, D) for l in range(w.layers)]
        kl_ = K.alloc_layers(cfgs, spl, n, dev, keys=True)
        vl_ = K.alloc_layers(cfgs, spl, n, dev, keys=False)
        k4, v4 = k.view(w.layers, spl, T, D), v.view(w.layers, spl, T, D)
        ko4, vo4 = ko.view(w.layers, spl, n, D), vo.view(w.layers, spl, n, D)
        calls = [
            lambda: K.kivi_encode_k_layers(cfgs, k4, n, kl_),
            lambda: K.kivi_encode_v_layers(cfgs, v4, n, vl_),
            lambda: K.kivi_decode_k_layers(cfgs, kl_, n, ko4),
            lambda: K.kivi_decode_v_layers(cfgs, vl_, n, vo4),
        ]
        for nm, keys in (("encode_k", True), ("encode_v", False), ("decode_k", True), ("decode_v", False)):
            sides = [(c.k_bits if keys else c.v_bits) for c in cfgs]
            launches[nm] = 1 + sum(1 for a, b in zip(sides, sides[1:]) if a != b)
    else:
        vq = K.alloc_values(cfg, S, n, dev)
    if w.fp8_keys:
        kq = torch.empty((S, n, D), dtype=torch.uint8, device=dev)
        calls = [
            lambda: K.kivi_fp8_encode(k, n, kq),
            lambda: K.kivi_encode_v(cfg, v, n, *vq),
            lambda: K.kivi_fp8_decode(kq, n, ko),
            lambda: K.kivi_decode_v(cfg, *vq, n, vo),
        ]
    elif not w.boundary:
        kq = K.alloc_keys(cfg, S, n, dev)
        calls = [
            lambda: K.kivi_encode_k(cfg, k, n, *kq),
            lambda: K.kivi_encode_v(cfg, v, n, *vq),
            lambda: K.kivi_decode_k(cfg, *kq, n, ko),
            lambda: K.kivi_decode_v(cfg, *vq, n, vo),
        ]
    ms_step, per_call, per_step = time_steps(calls, steps, args.warmup)
    per_kernel_ms = {nm: sum(per_call[j]) / steps for j, nm in enumerate(names)}
    per_kernel_med = {nm: _median(per_call[j]) for j, nm in enumerate(names)}

    fp16_eq = 2 * 2 * S * n * D * 2                  # K and V, encode + decode
    bits = {"encode_k": w.k_bits, "decode_k": w.k_bits, "encode_v": w.v_bits, "decode_v": w.v_bits}
    alg = {nm: algorithmic_bytes(nm[-1], nm[:6], S, n, D, G, bits[nm]) for nm in names}
    if w.boundary:                                    # each layer at its own bits
        alg = {nm: sum(algorithmic_bytes(nm[-1], nm[:6], spl, n, D, G,
                                         c.k_bits if nm[-1] == "k" else c.v_bits) for c in cfgs)
               for nm in names}
    if w.fp8_keys:                                    # 2 bytes in, 1 out (and back)
        alg["encode_k"] = alg["decode_k"] = 3 * S * n * D
    moved = sum(alg.values())
    dom = max(names, key=lambda nm: per_kernel_ms[nm])
    achieved = alg[dom] / (per_kernel_ms[dom] / 1000.0) / 1e9
    traffic = measured_traffic(dom, w_key(w))
    tokens = w.batch * n                              # sequence positions, all layers and heads
    med_step = _median(per_step)

    out = {
        "metric": "KV encode+decode GB/s (fp16-equivalent) and % of HBM roofline, 1 MI355X",
        "value": round(fp16_eq / (ms_step / 1000.0) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "layers": w.layers, "batch": w.batch, "kv_heads": w.heads, "head_dim": D,
            "seq_len": T, "quantized_tokens": n, "residual_length": w.residual_length,
            "k_bits": w.k_bits, "v_bits": w.v_bits, "group_size": G,
            "key_format": "fp8_e4m3" if w.fp8_keys else "kivi",
            **({"boundary_layers": sorted(prot), "boundary_bits": list(w.boundary_bits)} if w.boundary else {}),
        },
        "ms_per_step_median": round(med_step, 4),
        "moved_GBps": round(moved / (ms_step / 1000.0) / 1e9, 2),
        "hbm_roofline_frac_step": round(moved / (ms_step / 1000.0) / 1e9 / HBM_PEAK_GBPS, 4),
        "hbm_roofline_frac_step_median": round(moved / (med_step / 1000.0) / 1e9 / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(tokens / (ms_step / 1000.0), 1),
        "kernel_ms": {nm: round(x, 4) for nm, x in per_kernel_ms.items()},
        "kernel_ms_median": {nm: round(x, 4) for nm, x in per_kernel_med.items()},
        "kernel_GBps": {nm: round(alg[nm] / (per_kernel_ms[nm] / 1000.0) / 1e9, 1) for nm in names},
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg[dom] // launches[dom],
            **({"launches_per_call": launches[dom]} if launches[dom] > 1 else {}),
        },
    }
    if per_layer and not w.fp8_keys and not w.boundary:
        out["per_layer_loop"] = per_layer_bench(w, cfg, k, v, kq, vq, ko, vo, n, alg, steps, args.warmup)
    if attention and not w.fp8_keys and not w.boundary:
        out["attention"] = attention_bench(w, cfg, k, v, kq, vq, n, args, dev, cpu)
    if cpu:
        out["cpu_baseline"] = cpu_baseline(k, v, w, cfg, n, args.cpu_budget)
        out["cpu_baseline_all_cores"] = cpu_baseline_threads(k, v, w, cfg, n, args.cpu_budget)
    del k, v, ko, vo, kq, vq, calls
    torch.cuda.empty_cache()
    return out


def w_key(w):
    """The WORKLOADS key of a workload."""
    from kvsynth import WORKLOADS
    return next(key for key, x in WORKLOADS.items() if x is w)


def per_layer_bench(w, cfg, k, v, kq, vq, ko, vo, n, alg, steps, warmup):
    """The same step as a loop over layers: each kernel called once per layer
    (slices_per_layer slices a call), the way a model's cache is coded layer
    by layer; HIP events around each kernel's run of calls."""
    import kv_cache_quantization_codec_amd as K

    spl = w.slices_per_layer
    L = w.layers
    lay = [slice(l * spl, (l + 1) * spl) for l in range(L)]
    kql = [tuple(t[sl] for t in kq) for sl in lay]
    vql = [tuple(t[sl] for t in vq) for sl in lay]
    kl, vl, kol, vol = ([x[sl] for sl in lay] for x in (k, v, ko, vo))
    calls = [
        lambda: [K.kivi_encode_k(cfg, kl[l], n, *kql[l]) for l in range(L)],
        lambda: [K.kivi_encode_v(cfg, vl[l], n, *vql[l]) for l in range(L)],
        lambda: [K.kivi_decode_k(cfg, *kql[l], n, kol[l]) for l in range(L)],
        lambda: [K.kivi_decode_v(cfg, *vql[l], n, vol[l]) for l in range(L)],
    ]
    names = ["encode_k", "encode_v", "decode_k", "decode_v"]
    ms_step, per_call, per_step = time_steps(calls, steps, warmup)
    med = _median(per_step)
    moved = sum(alg.values())
    kms = {nm: _median(per_call[j]) for j, nm in enumerate(names)}
    slow = max(kms, key=kms.get)
    return {
        "what": f"the same step as {L} calls per kernel, one per layer of {spl} slices",
        "calls_per_kernel": L,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(med, 4),
        "kernel_ms_median": {nm: round(x, 4) for nm, x in kms.items()},
        "moved_GBps": round(moved / (med / 1000.0) / 1e9, 2),
        "hbm_roofline_frac_step": round(moved / (med / 1000.0) / 1e9 / HBM_PEAK_GBPS, 4),
        "slowest_kernel": slow,
        "slowest_kernel_frac": round(alg[slow] / (kms[slow] / 1000.0) / 1e9 / HBM_PEAK_GBPS, 4),
    }


def workload_summary(res: dict) -> dict:
    """The figures of a secondary workload's bench result kept on the main line."""
    keep = ("config", "ms_per_step", "ms_per_step_median", "value", "moved_GBps", "hbm_roofline_frac_step",
            "hbm_roofline_frac_step_median", "tokens_per_s", "kernel_ms_median", "kernel_GBps")
    out = {k: res[k] for k in keep if k in res}
    out["value_unit"] = "GB/s fp16-equivalent"
    out["slowest_kernel"] = res["roofline"]["kernel"]
    out["slowest_kernel_frac"] = res["roofline"]["frac"]
    if "attention" in res:
        a = res["attention"]
        out["attention"] = {k: a[k] for k in ("q_per_kv", "n_splits", "ms", "ms_runs", "algorithmic_bytes",
                                              "partial_sum_bytes", "achieved_GBps", "roofline_frac",
                                              "fp16_cache_equiv_GBps") if k in a}
    return out


def latency_bench(w, args, dev, reps=200):
    """A cache too small to stream (the single-layer workload): the step's
    latency in microseconds, median over ``reps`` steps."""
    import kv_cache_quantization_codec_amd as K

    cfg = K.Config(w.k_bits, w.v_bits, w.group_size, w.residual_length, w.head_dim)
    S, D = w.slices, w.head_dim
    n = w.tokens - w.residual_length
    k, v = build_cache(w, dev)
    kq, vq = K.alloc_keys(cfg, S, n, dev), K.alloc_values(cfg, S, n, dev)
    ko, vo = k.new_empty((S, n, D)), v.new_empty((S, n, D))
    calls = [lambda: K.kivi_encode_k(cfg, k, n, *kq), lambda: K.kivi_encode_v(cfg, v, n, *vq),
             lambda: K.kivi_decode_k(cfg, *kq, n, ko), lambda: K.kivi_decode_v(cfg, *vq, n, vo)]
    _, per_call, per_step = time_steps(calls, reps, 20)
    names = ["encode_k", "encode_v", "decode_k", "decode_v"]
    moved = sum(algorithmic_bytes(nm[-1], nm[:6], S, n, D, w.group_size, w.k_bits if nm[-1] == "k"
                                  else w.v_bits) for nm in names)
    return {
        "config": {"workload": w.name, "slices": S, "seq_len": w.tokens, "quantized_tokens": n,
                   "k_bits": w.k_bits, "v_bits": w.v_bits, "group_size": w.group_size},
        "us_per_step_median": round(_median(per_step) * 1000.0, 2),
        "kernel_us_median": {nm: round(_median(per_call[j]) * 1000.0, 2) for j, nm in enumerate(names)},
        "moved_bytes": moved,
        "steps": reps,
        "note": "latency bound: 4 MB moved per step, below a kernel launch's cost",
    }


def stream_summary(res: dict) -> dict:
    keep = ("config", "value", "unit", "p99_us", "flush_steps", "flush_p50_us", "flush_p99_us",
            "append_p50_us", "append_p99_us", "append_GBps", "flush_GBps", "prefill_ms", "prefill_GBps",
            "final_state", "offload_restore")
    out = {k: res[k] for k in keep if k in res}
    out["value_is"] = "p50 step latency over all steps"
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama2_7b_2bit",
                    choices=["llama2_7b_2bit", "mistral_7b_k2v4", "single_layer_4bit",
                             "llama2_7b_k8v4", "llama2_7b_mix", "stream_b64"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the chosen workload (no per-layer loop, secondary workloads "
                         "or copy ceiling): for profiler runs")
    ap.add_argument("--copy-ceiling", action="store_true",
                    help="also time a plain 4 GiB device-to-device copy (always done in the default run)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.txt from two rocprofv3 --pmc "
                         "counter_collection CSVs of this script and exit (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_traffic:
        text = summarize_traffic(args.workload, *args.summarize_traffic)
        path = os.path.join(ROOT, "profiles", f"traffic_{args.workload}.txt")
        with open(path, "w") as f:
            f.write(text)
        print(text, end="")
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this codec benchmark runs on one GPU only; "
                                   "--gpus must be 1 (slices shard across GPUs with no exchange, "
                                   "so per-GPU throughput is the figure)"}), flush=True)
        sys.exit(2)

    import torch

    import kv_cache_quantization_codec_amd as K
    from kvsynth import WORKLOADS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    K.binding.lib()
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.workload]
    if w.steps:
        print(json.dumps(stream_bench(w, args)), flush=True)
        return
    full = args.workload == "llama2_7b_2bit" and not args.headline_only
    cpu = not args.no_cpu_baseline
    out = codec_bench(w, args, dev, attention=True, cpu=cpu, per_layer=full)
    if full:
        # the other workloads of the same measurement, each after the previous
        # one's device memory is released
        out["mistral_7b_k2v4"] = workload_summary(
            codec_bench(WORKLOADS["mistral_7b_k2v4"], args, dev, attention=True, cpu=False))
        out["single_layer_4bit"] = latency_bench(WORKLOADS["single_layer_4bit"], args, dev)
        out["stream_b64"] = stream_summary(stream_bench(WORKLOADS["stream_b64"], args))
    if full or args.copy_ceiling:
        out["copy_ceiling_GBps"] = copy_ceiling(dev)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
