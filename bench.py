#!/usr/bin/env python3
"""Benchmark of the paged MLA decode hot path on one MI355X.

One step = the whole path over one batch of synthetic input: the split-KV
metadata call (mla_get_metadata), the main kernel (mla_decode_splitkv) and
the split combine (mla_decode_combine), all on the current stream.

The metric has two halves, and the default run measures both:
  * "membound" (the memory-bound half, HBM TB/s at h_q=16): B=32, s_q=1,
    h_q=16, h_kv=1, every N=4096; its figures are the line's top-level
    value / roofline;
  * "mtp" (the compute-bound half, TFLOPS at h_q=128): B=64, s_q=2 causal,
    h_q=128, N ~ U{1024..8192}; its figures are under "compute_bound", with a
    roofline against the bf16 MFMA peak.
Page 64, bf16 N(0,1) data, scale 576^-0.5.  Inputs are resident in HBM before
the timed region; every step reads a different copy of the KV pool (copies
rotate over >= 1 GiB) so that the 256 MB Infinity Cache cannot serve the
pool from the previous step.  --workload W measures only W.

Output: one JSON line on stdout (details on stderr).
  value       algorithmic bytes per step / time per step (TB/s); bytes =
              every visible KV row once + q + out + lse + needed table entries
              + cache_seqlens (no padding, re-reads or split partials)
  roofline    the main decode kernel alone: algorithmic bytes per launch /
              its mean duration (HIP events on the launch stream around
              max(K, 200) back-to-back launches), against 8 TB/s (or its flops against
              2.5 PFLOP/s bf16 for MFMA-bound workloads); traffic = HBM bytes
              per launch from the committed rocprofv3 counter summary when it
              matches the current kernel source, else null
  gpu_torch_baseline  plain PyTorch on the GPU, same inputs (context)
  cpu_baseline  the CPU oracle (fp64, OpenMP) on the primary workload
  oracle_parity  the timed step's whole output against the oracle

Profile summaries: `--summarize-profiles DIR` turns the rocprofv3 output that
the commands below leave in DIR into the text summaries and the counter file
under profiles/ (run from /tmp, TMPDIR=/tmp; WL = membound, mtp, large,
ragged or hkv2):
  rocprofv3 --kernel-trace --stats -d DIR/trace_WL -o run --output-format csv
      -- python3 /root/repo/bench.py --workload WL --steps 100 --warmup 10 --no-cpu-baseline --no-torch-baseline --no-ceilings
  rocprofv3 --pmc FETCH_SIZE -d DIR/pmc_FETCH_SIZE_WL -o run --output-format csv
      -- python3 /root/repo/bench.py --workload WL --steps 5 --warmup 2 --no-cpu-baseline --no-torch-baseline --no-ceilings
  (the same with WRITE_SIZE), and both counters once more with
      -- python3 /root/repo/bench.py --copy-calibration   (dirs pmc_FETCH_SIZE_copy, ...)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

SIMDS = 256 * 4  # MI355X: 256 CUs of 4 SIMDs
XCDS = 8
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
COUNTERS = os.path.join(ROOT, "profiles", "decode_kernel_counters.json")
METRIC = "paged MLA decode: achieved HBM TB/s (h_q=16) and TFLOPS (h_q=128)"


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_units(w):
    """Bytes and flops the method must move / compute for one call."""
    n = w.seqlens.astype(np.int64)
    B = n.shape[0]
    pages = int(((n + 63) // 64).sum())
    rows = B * w.s_q * w.h_q
    nbytes = int(n.sum()) * w.h_kv * 576 * 2 + rows * (576 * 2 + 512 * 2 + 4) + pages * 4 + B * 4
    pairs = 0
    for t in range(w.s_q):
        vis = np.minimum(n, n - w.s_q + t + 1) if w.causal else n
        pairs += int(np.clip(vis, 0, None).sum())
    flops = 2 * (576 + 512) * pairs * w.h_q
    return nbytes, flops


def kernel_source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mla_decode_attention_split_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")) and name != "ceiling.hip":
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def counter_traffic(workload):
    """HBM bytes per launch of the decode kernel from the committed counter
    summary, if it was taken on this workload with the current source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    entry = c.get("workloads", {}).get(workload)
    if not entry or c.get("kernel_source_digest") != kernel_source_digest():
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(w, min_seconds=10.0):
    import oracle
    oracle.build(force=False)
    nbytes, flops = algorithmic_units(w)
    times = []
    t_end = time.perf_counter() + min_seconds
    while time.perf_counter() < t_end or len(times) < 3:
        t0 = time.perf_counter()
        oracle.decode(w.q, w.kcache, w.block_table, w.seqlens, causal=w.causal, scale=w.scale,
                      dtype=w.dtype)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return {"value": nbytes / med / 1e12, "unit": "TB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "tflops": flops / med / 1e12,
            "sample": f"whole {w.name} workload ({w.batch} sequences), median of {len(times)} "
                      f"runs of {med:.3f} s, fp64"}


def torch_baseline(w, q, kv, bt, steps=10):
    """Plain PyTorch on the GPU, for context (the pages compare FlashMLA with a
    native Torch implementation): gather every sequence's pages into a padded
    dense K (B, Nmax, 576), scores as one batched 16-bit product, masked
    softmax in fp32, P (rounded to q's type) times V.  One KV head only.
    Every operand of a batched product is made contiguous first.

    Returns (ms per call, out [B, s_q, h_q, 512] in q's type, lse fp32
    [B, s_q, h_q])."""
    import torch
    B, s_q, h_q = w.batch, w.s_q, w.h_q
    M = s_q * h_q
    n = torch.from_numpy(w.seqlens.astype(np.int64)).to(q.device)
    pmax = max(1, int((int(w.seqlens.max()) + 63) // 64))
    jj = torch.arange(pmax * 64, device=q.device)
    row_t = torch.arange(M, device=q.device) // h_q
    lim = n[:, None] - s_q + row_t[None, :] + 1 if w.causal else n[:, None].expand(B, M)
    lim = torch.minimum(lim, n[:, None])
    masked = jj[None, :, None] >= lim[:, None, :]                       # (B, Nmax, M)
    pages = kv.view(kv.shape[0], 64, 576)

    def run():
        K = pages[bt[:, :pmax].long()].reshape(B, pmax * 64, 576)        # gather
        qT = q.reshape(B, M, 576).transpose(1, 2).contiguous()             # (B, 576, M)
        St = torch.bmm(K, qT).float() * w.scale                            # (B, Nmax, M)
        St = St.masked_fill(masked, float("-inf"))
        lse = torch.logsumexp(St, dim=1)                                   # (B, M)
        P = torch.exp(St - lse[:, None, :]).transpose(1, 2).contiguous().to(q.dtype)
        V = K[:, :, :512].contiguous()
        return torch.bmm(P, V), lse                                        # (B, M, 512)

    o, l = run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return ms, o.reshape(B, s_q, h_q, 512), l.reshape(B, s_q, h_q)


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _per_kernel_counter(path):
    """Mean counter value (KiB) per dispatch, per kernel name."""
    acc = {}
    for r in _csv_rows(path):
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def _short_kernel(name):
    if "spin_kernel" in name:
        return "torch spin_kernel (stream hold before timed passes)"
    return name.split("(unsigned")[0].split("(int")[0].split("(mla::")[0].replace("void ", "")


def summarize_profiles(d):
    """Write profiles/<kernel>_<workload>.txt and profiles/decode_kernel_counters.json."""
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    # Calibration: a plain 1 GiB device copy reads and writes 1 GiB.
    copy_bytes = float(1 << 30) * 5
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        k = _per_kernel_counter(os.path.join(d, f"pmc_{c}_copy", "run_counter_collection.csv"))
        copy = [(v, n) for name, (v, n) in k.items() if "copyBuffer" in name]
        tot = sum(v * n for v, n in copy) * 1024.0
        cal[c] = {"measured_bytes": tot, "true_bytes": copy_bytes, "scale": copy_bytes / tot}
    # The digest of the source the profiled runs measured (each run prints it),
    # so that summaries of older runs are never stamped with a newer digest.
    import re
    seen = set()
    for wl in ("membound", "mtp", "large", "ragged", "hkv2"):
        ep = os.path.join(d, f"trace_{wl}.err")
        if os.path.exists(ep):
            seen |= set(re.findall(r"kernel source digest ([0-9a-f]{16})", open(ep).read()))
    if len(seen) != 1:
        raise SystemExit(f"profiled runs name {len(seen)} kernel source digests ({sorted(seen)}); "
                         f"profile every workload with one build")
    run_digest = seen.pop()
    if run_digest != kernel_source_digest():
        eprint(f"note: the profiled source ({run_digest}) is not the current source "
               f"({kernel_source_digest()}); the bench will not use these counters")
    counters = {"kernel_source_digest": run_digest,
                "calibration": {"kernel": "__amd_rocclr_copyBuffer (torch copy_ of 1 GiB, x5)",
                                "fetch_scale": round(cal["FETCH_SIZE"]["scale"], 4),
                                "write_scale": round(cal["WRITE_SIZE"]["scale"], 4)},
                "workloads": {}}
    for wl in ("membound", "mtp", "large", "ragged", "hkv2"):
        tdir = os.path.join(d, f"trace_{wl}")
        if not os.path.isdir(tdir):
            continue
        stats = _csv_rows(os.path.join(tdir, "run_kernel_stats.csv"))
        fetch = _per_kernel_counter(os.path.join(d, f"pmc_FETCH_SIZE_{wl}", "run_counter_collection.csv"))
        write = _per_kernel_counter(os.path.join(d, f"pmc_WRITE_SIZE_{wl}", "run_counter_collection.csv"))
        import re
        bench_err = [x for x in open(os.path.join(d, f"trace_{wl}.err")).read().strip().splitlines()
                     if not re.match(r"^[WEI]\d{8} ", x)]
        lines = [f"# rocprofv3 kernel trace: paged MLA decode, workload {wl}", "",
                 "command (from /tmp, TMPDIR=/tmp):",
                 f"  rocprofv3 --kernel-trace --stats -d DIR/trace_{wl} -o run --output-format csv "
                 f"-- python3 /root/repo/bench.py --workload {wl} --steps 100 --warmup 10 --no-cpu-baseline --no-torch-baseline --no-ceilings",
                 f"kernel source digest: {counters['kernel_source_digest']}", "",
                 f"{'kernel':60s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s}"]
        for r in stats:
            name = _short_kernel(r["Name"])
            lines.append(f"{name[:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                         f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}")
        lines += ["", "bench.py stderr under the profiler:"] + ["  " + x for x in bench_err]
        lines += ["", "HBM counters (separate runs, --steps 5 --warmup 2; KiB per dispatch, raw):"]
        entry = None
        for name, (fv, n) in fetch.items():
            wv = write.get(name, (float("nan"), 0))[0]
            short = _short_kernel(name)
            lines.append(f"  {short[:58]:58s} FETCH_SIZE {fv:12.1f}  WRITE_SIZE {wv:12.1f}  ({n} dispatches)")
            if "decode_kernel" in name:
                fb = fv * 1024 * cal["FETCH_SIZE"]["scale"]
                wb = wv * 1024 * cal["WRITE_SIZE"]["scale"]
                entry = {"kernel": short, "fetch_kib_raw": round(fv, 1), "write_kib_raw": round(wv, 1),
                         "hbm_read_bytes_per_launch": int(fb), "hbm_write_bytes_per_launch": int(wb),
                         "hbm_bytes_per_launch": int(fb + wb)}
        if entry:
            counters["workloads"][wl] = entry
            lines += ["", f"copy calibration: FETCH_SIZE x{cal['FETCH_SIZE']['scale']:.4f}, "
                          f"WRITE_SIZE x{cal['WRITE_SIZE']['scale']:.4f} (1 GiB torch copy read/written 5 times)",
                      f"decode kernel HBM bytes per launch: read {entry['hbm_read_bytes_per_launch'] / 1e6:.2f} MB, "
                      f"write {entry['hbm_write_bytes_per_launch'] / 1e6:.2f} MB"]
        sq_path = os.path.join(d, f"pmc_SQ_{wl}", "run_counter_collection.csv")
        if os.path.exists(sq_path):
            per = {}
            for r in _csv_rows(sq_path):
                if "decode_kernel" in r["Kernel_Name"]:
                    per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            mean = {k: sum(v) / len(v) for k, v in per.items()}
            lines += ["", "SQ counters of the decode kernel (separate run, --steps 5 --warmup 2; mean per "
                          "dispatch):",
                      f"  command: rocprofv3 --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES "
                      f"SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS SQ_WAIT_INST_ANY "
                      f"SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE -d DIR/pmc_SQ_{wl} -o run --output-format csv -- "
                      f"python3 /root/repo/bench.py --workload {wl} --steps 5 --warmup 2 --no-cpu-baseline --no-torch-baseline --no-ceilings"]
            for k in sorted(mean):
                lines.append(f"  {k:28s} {mean[k]:16.1f}")
            if mean.get("GRBM_GUI_ACTIVE") and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                # GRBM_GUI_ACTIVE is summed over the XCDs; SQ_VALU_MFMA_BUSY_CYCLES over all
                # SIMDs (it reads 32 cycles per 32x32x16 MFMA).
                active = mean["GRBM_GUI_ACTIVE"] / XCDS
                util = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * SIMDS)
                lines.append(f"  MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCDS} "
                             f"XCDs x {SIMDS} SIMDs) = {util:.3f}")
                dec = [r for r in stats if "decode_kernel" in r["Name"]]
                if dec:
                    ns = float(dec[0]["AverageNs"])
                    lines.append(f"  GRBM_GUI_ACTIVE / {XCDS} / mean kernel time ({ns / 1e3:.2f} us, kernel "
                                 f"trace) = {active / ns:.2f} GHz (the counter window also spans the "
                                 f"dispatch, so for short kernels this overstates the shader clock and "
                                 f"understates the MFMA busy fraction)")
                if mean.get("SQ_WAVE_CYCLES") and mean.get("SQ_WAVES"):
                    # SQ_WAVE_CYCLES counts in units of 4 cycles; every tile runs one wave per SIMD
                    wave_cyc = 4.0 * mean["SQ_WAVE_CYCLES"]
                    util_w = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / wave_cyc
                    lines.append(f"  MFMA busy while a wave is resident = SQ_VALU_MFMA_BUSY_CYCLES / (4 x "
                                 f"SQ_WAVE_CYCLES) = {util_w:.3f} (one wave per SIMD)")
                    if dec:
                        per_wave = wave_cyc / mean["SQ_WAVES"]
                        lines.append(f"  cycles per wave = 4 x SQ_WAVE_CYCLES / SQ_WAVES = {per_wave:.0f}; over the "
                                     f"mean kernel time: {per_wave / ns:.2f} GHz (a lower bound of the shader "
                                     f"clock: waves live shorter than the kernel)")
                    if entry:
                        entry["mfma_busy_frac_resident"] = round(util_w, 4)
                if entry:
                    entry["mfma_busy_frac"] = round(util, 4)
            if mean.get("SQ_INSTS_LDS"):
                lines.append(f"  LDS bank-conflict cycles per LDS instruction = "
                             f"{mean.get('SQ_LDS_BANK_CONFLICT', 0.0) / mean['SQ_INSTS_LDS']:.4f}")
        with open(os.path.join(out_dir, f"decode_kernel_{wl}.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
    clocks = os.path.join(d, "clocks.txt")
    if os.path.exists(clocks):
        keep = [x for x in open(clocks).read().splitlines() if "clk" in x.lower() or "GPU[" in x]
        with open(os.path.join(out_dir, "gpu_clocks.txt"), "w") as f:
            f.write("# rocm-smi --showclocks on the GPU box, idle, before the profiled runs (the clock under\n"
                    "# load is derived from counters in decode_kernel_<workload>.txt)\n")
            f.write("\n".join(keep) + "\n")
    with open(COUNTERS, "w") as f:
        json.dump(counters, f, indent=1)
        f.write("\n")
    print(json.dumps(counters, indent=1))


def ceiling_lib():
    """The measurement library (libmla_ceiling.so, include/mla_ceiling.h)."""
    global _CEILING
    if _CEILING is None:
        import ctypes
        import mla_decode_attention_split_amd as mla
        path = os.path.join(os.path.dirname(mla.library_path()), "libmla_ceiling.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m mla_decode_attention_split_amd.build`")
        lib = ctypes.CDLL(path)
        p, i = ctypes.c_void_p, ctypes.c_int
        lib.mla_ceiling_stream.argtypes = [p, i, i, p, i, i, p, p]
        lib.mla_ceiling_stream.restype = i
        lib.mla_ceiling_mfma.argtypes = [p, i, i, i, p]
        lib.mla_ceiling_mfma.restype = i
        lib.mla_ceiling_last_error.restype = ctypes.c_char_p
        _CEILING = lib
    return _CEILING


_CEILING = None


def _ceiling_check(rc):
    if rc != 0:
        raise RuntimeError(f"ceiling probe failed [{rc}]: {ceiling_lib().mla_ceiling_last_error().decode()}")


def _stream_ptr(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def ceiling_stream(pool, pages, sink):
    """Stream the cache pages listed in ``pages`` (int32 [workgroups,
    pages_per_workgroup]) of ``pool`` ([num_pages, 64 * 576] 16-bit) through
    the decode kernel's LDS ring, no arithmetic."""
    W, P = pages.shape
    _ceiling_check(ceiling_lib().mla_ceiling_stream(
        pool.data_ptr(), int(pool.shape[0]), pool[0].numel() * pool.element_size(), pages.data_ptr(),
        int(W), int(P), sink.data_ptr(), _stream_ptr(pool)))


def ceiling_mfma(sink, num_workgroups, iters, random_operands=False):
    """num_workgroups x 4 waves of iters x 4 independent 32x32x16 bf16 MFMAs,
    on constant operands or on random operands that change every MFMA."""
    _ceiling_check(ceiling_lib().mla_ceiling_mfma(sink.data_ptr(), int(num_workgroups), int(iters),
                                                  int(bool(random_operands)), _stream_ptr(sink)))


def span_ms(fn, k, hold_cycles=int(2.4e9 * 0.005)):
    """Mean duration of k back-to-back calls of fn(i), HIP events on the
    current stream at both ends, the stream held by a spin while they are
    enqueued."""
    import torch
    a0 = torch.cuda.Event(enable_timing=True)
    a1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(hold_cycles)
    a0.record()
    for i in range(k):
        fn(i)
    a1.record()
    torch.cuda.synchronize()
    return a0.elapsed_time(a1) / k


def measure_workload(name, args, dev, primary):
    """Time one workload's step and its parts; returns (block, w, out, lse)."""
    import torch
    import mla_decode_attention_split_amd as mla
    from mla_decode_attention_split_amd import synth

    w = synth.named_workload(name, dtype=args.dtype)
    nbytes, flops = algorithmic_units(w)
    M, h_kv = w.rows_per_kv_head, w.h_kv
    eprint(f"[{name}] kernel source digest {kernel_source_digest()}")
    pool_bytes = w.kcache.nbytes
    copies = max(1, int(np.ceil(args.rotate_bytes / pool_bytes)))
    eprint(f"[{name}] B={w.batch} s_q={w.s_q} h_q={w.h_q} h_kv={h_kv} causal={w.causal} "
           f"sum(N)={int(w.seqlens.sum())} bytes={nbytes / 1e6:.2f} MB flops={flops / 1e9:.2f} GFLOP "
           f"pool={pool_bytes / 1e6:.1f} MB x{copies} copies")

    tdt = torch.float16 if args.dtype == "fp16" else torch.bfloat16
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(tdt)
    kv0 = torch.from_numpy(w.kcache.view(np.int16)).to(dev).view(tdt)
    kvs = [kv0] + [kv0.clone() for _ in range(copies - 1)]
    bt = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
    sl = torch.from_numpy(np.ascontiguousarray(w.seqlens)).to(dev)
    num_parts, _ = mla.mla_metadata_shape(w.batch, M, h_kv)
    tile_rows, m_tiles, fixed_cost = mla.mla_tile_shape(M, h_kv)
    meta = torch.empty((num_parts, 8), dtype=torch.int32, device=dev)
    splits = torch.empty((w.batch + 1,), dtype=torch.int32, device=dev)
    out = torch.empty((w.batch, w.s_q, w.h_q, 512), dtype=tdt, device=dev)
    lse = torch.empty((w.batch, w.s_q, w.h_q), dtype=torch.float32, device=dev)
    ws = torch.empty((mla.mla_workspace_bytes(w.batch, M, h_kv, num_parts),), dtype=torch.uint8,
                     device=dev)
    eprint(f"[{name}] num_parts={num_parts} fixed_cost={fixed_cost} tile_rows={tile_rows} "
           f"grid={num_parts * m_tiles * h_kv}")

    def step(i):
        mla.mla_get_metadata(sl, M, h_kv, tile_metadata=meta, num_splits=splits)
        mla.mla_decode_splitkv(q, kvs[i % copies], bt, sl, meta, splits, causal=w.causal,
                               softmax_scale=w.scale, out=out, lse=lse, workspace=ws)
        mla.mla_decode_combine(splits, out, lse, ws, num_parts=num_parts, h_kv=h_kv)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Host enqueue rate, to size the spin that holds the stream while the
    # timed steps are queued (so the GPU then runs them back to back).
    t0 = time.perf_counter()
    for i in range(20):
        step(i)
    enqueue_s = (time.perf_counter() - t0) / 20
    torch.cuda.synchronize()
    hold_cycles = int(2.4e9 * (1.5 * enqueue_s * args.steps + 0.01))

    # Pass 1: throughput of whole steps (events only at the ends).
    ms_per_step = span_ms(step, args.steps, hold_cycles)

    # The timed step's result, checked bitwise against one mla_decode call on
    # the same inputs (the two launches of the step are the decode's halves).
    step(0)
    out_chk = torch.empty_like(out)
    lse_chk = torch.empty_like(lse)
    mla.mla_decode(q, kvs[0], bt, sl, meta, splits, causal=w.causal, softmax_scale=w.scale,
                   out=out_chk, lse=lse_chk)
    torch.cuda.synchronize()
    same = bool(torch.equal(out.view(torch.int16), out_chk.view(torch.int16)) and
                torch.equal(lse.view(torch.int32), lse_chk.view(torch.int32)))
    out_np = out.float().cpu().numpy().astype(np.float64)
    lse_np = lse.cpu().numpy().astype(np.float64)

    # Pass 2: the main kernel alone, launched back to back over the same
    # metadata (computed once, outside the timed region), HIP events at both
    # ends on the stream the kernel runs on; mean launch duration = span / K.
    # K is at least 200 launches: the chip's clock under load settles over
    # milliseconds (it is power-limited), and a short window would weigh the
    # first launches after the idle hold too much.
    k_dec = max(args.steps, 200)
    hold_dec = int(2.4e9 * (1.5 * enqueue_s * k_dec + 0.01))
    dec_ms = span_ms(lambda i: mla.mla_decode_splitkv(q, kvs[i % copies], bt, sl, meta, splits,
                                                      causal=w.causal, softmax_scale=w.scale,
                                                      out=out, lse=lse, workspace=ws),
                     k_dec, hold_dec)
    # Pass 3: the metadata call and the combine alone (same buffers).
    meta_ms = span_ms(lambda i: mla.mla_get_metadata(sl, M, h_kv, tile_metadata=meta,
                                                     num_splits=splits), 200)
    comb_ms = span_ms(lambda i: mla.mla_decode_combine(splits, out, lse, ws, num_parts=num_parts,
                                                       h_kv=h_kv), 200)

    hbm_bound = name != "mtp"
    step_tbs = nbytes / (ms_per_step * 1e-3) / 1e12
    step_tflops = flops / (ms_per_step * 1e-3) / 1e12
    if hbm_bound:
        achieved = nbytes / (dec_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = flops / (dec_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof["traffic"] = counter_traffic(name)
    eprint(f"[{name}] host enqueue {enqueue_s * 1e6:.1f} us/step")
    eprint(f"[{name}] step {ms_per_step * 1e3:.2f} us -> {step_tbs:.3f} TB/s, {step_tflops:.1f} TFLOP/s")
    eprint(f"[{name}] decode kernel {dec_ms * 1e3:.2f} us mean over {k_dec} back-to-back launches "
           f"-> {achieved:.1f} {roof['unit']} ({roof['frac'] * 100:.1f}% of peak)")
    eprint(f"[{name}] metadata call {meta_ms * 1e3:.2f} us, combine {comb_ms * 1e3:.2f} us (each alone); "
           f"timed step equals mla_decode bitwise: {same}")

    block = {
        "workload": name,
        "config": {"workload": w.name, "batch": w.batch, "s_q": w.s_q, "h_q": w.h_q,
                   "h_kv": h_kv, "seqlens_sum": int(w.seqlens.sum()), "page": 64, "d": 576,
                   "dv": 512, "causal": bool(w.causal), "kv_pool_copies": copies,
                   "num_parts": num_parts, "tile_rows": tile_rows},
        "ms_per_step": round(ms_per_step, 5),
        "tbs": round(step_tbs, 4),
        "tflops": round(step_tflops, 3),
        "decode_kernel_us": round(dec_ms * 1e3, 3),
        "decode_kernel_launches": k_dec,
        "roofline": roof,
        "parts_us": {"metadata": round(meta_ms * 1e3, 3), "decode": round(dec_ms * 1e3, 3),
                     "combine": round(comb_ms * 1e3, 3)},
        "step_equals_mla_decode": same,
    }
    if not args.no_torch_baseline and h_kv == 1:
        t_ms, t_out, _ = torch_baseline(w, q, kvs[0], bt)
        t_diff = float((t_out.float().reshape(out_chk.shape) - out_chk.float()).abs().max().item())
        block["gpu_torch_baseline"] = {
            "value": round(nbytes / (t_ms * 1e-3) / 1e12, 4), "unit": "TB/s",
            "tflops": round(flops / (t_ms * 1e-3) / 1e12, 2), "ms": round(t_ms, 4),
            "max_abs_diff_vs_kernel": t_diff,
            "what": "PyTorch on the GPU: padded dense gather of the pages, bf16 batched products, "
                    "fp32 masked softmax; pool already warm in cache"}
        eprint(f"[{name}] torch baseline {t_ms * 1e3:.1f} us per call "
               f"({nbytes / (t_ms * 1e-3) / 1e12:.3f} TB/s, {flops / (t_ms * 1e-3) / 1e12:.1f} TFLOP/s), "
               f"max |diff| vs kernel {t_diff:.3g}")
        del t_out
    ctx = {"w": w, "kvs": kvs, "hbm_bound": hbm_bound, "achieved": achieved, "nbytes": nbytes,
           "flops": flops, "out": out_np, "lse": lse_np, "copies": copies}
    return block, ctx


def oracle_parity(ctx):
    """The GPU step's whole out / lse against the oracle (test infrastructure),
    with the tolerance the tests use."""
    import oracle
    w = ctx["w"]
    ro, rl = oracle.decode(w.q, w.kcache, w.block_table, w.seqlens, causal=w.causal, scale=w.scale,
                           dtype=w.dtype)
    d = ctx["out"] - ro
    fin = np.isfinite(rl)
    res = {"out_max_abs": float(np.abs(d).max()),
           "out_rel_fro": float(np.linalg.norm(d) / max(np.linalg.norm(ro), 1e-300)),
           "lse_max_abs": float(np.abs(ctx["lse"][fin] - rl[fin]).max()) if fin.any() else 0.0}
    res["within_tolerance"] = bool(res["out_max_abs"] <= 2e-2 and res["out_rel_fro"] <= 5e-3 and
                                   res["lse_max_abs"] <= 1e-3)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None,
                    choices=["tiny", "membound", "mtp", "large", "ragged", "hkv2"],
                    help="measure only this workload (default: membound, plus mtp as the "
                         "compute-bound half of the metric)")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp16"],
                    help="element type of q, the cache and out")
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 30),
                    help="total bytes of KV pool copies the steps rotate over")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle (CPU baseline timing and the parity check)")
    ap.add_argument("--no-torch-baseline", action="store_true",
                    help="skip the plain PyTorch implementation on the GPU (context)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured ceilings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM counters)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 output in DIR and exit")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); this path has no multi-GPU leg.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        eprint("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        eprint(f"copied {n} bytes x 5")
        return

    primary_name = args.workload or "membound"
    block, ctx = measure_workload(primary_name, args, dev, primary=True)
    second = None
    if args.workload is None:
        second, ctx2 = measure_workload("mtp", args, dev, primary=False)

    # Ceilings measured on this GPU: (a) the pages the primary workload reads,
    # streamed through the main kernel's LDS ring with no arithmetic, over the
    # same rotating pool copies; (b) a loop of independent bf16 MFMAs on every
    # SIMD.
    ceilings = None
    if not args.no_ceilings:
        w = ctx["w"]
        used = [p for b in range(w.batch) for p in w.block_table[b, :(int(w.seqlens[b]) + 63) // 64]]
        groups = 256
        per = max(1, (len(used) + groups - 1) // groups)
        plist = np.full(groups * per, w.kcache.shape[0], dtype=np.int32)  # padding: outside the pool
        plist[:len(used)] = np.asarray(used, dtype=np.int32)
        pages_t = torch.from_numpy(plist.reshape(groups, per)).to(dev)
        isink = torch.zeros(1, dtype=torch.int32, device=dev)
        fsink = torch.zeros(1, dtype=torch.float32, device=dev)
        stream_tbs = None
        if w.h_kv == 1:  # the ring streams pages of one KV head
            kv_pages = [kc.view(kc.shape[0], -1) for kc in ctx["kvs"]]
            copies = ctx["copies"]
            for i in range(3):
                ceiling_stream(kv_pages[i % copies], pages_t, isink)
            stream_ms = span_ms(lambda i: ceiling_stream(kv_pages[i % copies], pages_t, isink), 100)
            stream_tbs = len(used) * 64 * 1152 / (stream_ms * 1e-3) / 1e12
        mf_wg, mf_it = 1024, 1000
        ceiling_mfma(fsink, mf_wg, mf_it)
        mfma_ms = span_ms(lambda i: ceiling_mfma(fsink, mf_wg, mf_it), 20)
        mfma_tflops = mf_wg * 4 * mf_it * 4 * 32768 / (mfma_ms * 1e-3) / 1e12
        ceiling_mfma(fsink, mf_wg, mf_it, True)
        mfma_r_ms = span_ms(lambda i: ceiling_mfma(fsink, mf_wg, mf_it, True), 20)
        mfma_r_tflops = mf_wg * 4 * mf_it * 4 * 32768 / (mfma_r_ms * 1e-3) / 1e12
        ceilings = {
            "stream_read": None if stream_tbs is None else {
                "value": round(stream_tbs, 4), "unit": "TB/s",
                "what": f"the {primary_name} workload's cache pages through the main kernel's LDS "
                        f"ring, no arithmetic, rotating pool copies"},
            "mfma_bf16": {"value": round(mfma_tflops, 1), "unit": "TFLOP/s",
                          "what": "independent 32x32x16 bf16 MFMA chains on every SIMD, constant operands"},
            "mfma_bf16_random": {"value": round(mfma_r_tflops, 1), "unit": "TFLOP/s",
                                 "what": "the same on random bf16 operands that change every MFMA "
                                         "(the switching power lowers the clock the chip holds)"},
        }
        ceil_p = (stream_tbs * 1e3 if stream_tbs else None) if ctx["hbm_bound"] else mfma_tflops
        ceilings["decode_frac"] = round(ctx["achieved"] / ceil_p, 4) if ceil_p else None
        if second is not None:
            ceilings["compute_bound_decode_frac"] = round(ctx2["achieved"] / mfma_tflops, 4)
            ceilings["compute_bound_decode_frac_random"] = round(ctx2["achieved"] / mfma_r_tflops, 4)
        eprint(f"measured ceilings: paged stream {stream_tbs} TB/s, bf16 MFMA loop {mfma_tflops:.1f} TFLOP/s "
               f"(random operands {mfma_r_tflops:.1f} TFLOP/s)")
        for key, c in (("primary", ctx), ("compute-bound", ctx2 if second is not None else None)):
            if c is not None:
                cp = (stream_tbs * 1e3 if stream_tbs else None) if c["hbm_bound"] else mfma_tflops
                if cp:
                    eprint(f"{key} decode kernel at {c['achieved'] / cp * 100:.1f}% of the measured "
                           f"{'stream' if c['hbm_bound'] else 'MFMA'} ceiling")

    hbm_bound = ctx["hbm_bound"]
    result = {
        "metric": METRIC,
        "value": block["tbs"] if hbm_bound else block["tflops"],
        "unit": "TB/s" if hbm_bound else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": block["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": block["config"],
        "tflops": block["tflops"],
        "decode_kernel_us": block["decode_kernel_us"],
        "decode_kernel_launches": block["decode_kernel_launches"],
        "roofline": block["roofline"],
        "parts_us": block["parts_us"],
        "step_equals_mla_decode": block["step_equals_mla_decode"],
    }
    if "gpu_torch_baseline" in block:
        result["gpu_torch_baseline"] = block["gpu_torch_baseline"]
    if second is not None:
        result["compute_bound"] = second
    if ceilings is not None:
        result["measured_ceilings"] = ceilings
    if not args.no_cpu_baseline:
        eprint("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(ctx["w"])
        eprint(f"cpu baseline {result['cpu_baseline']}")
        result["oracle_parity"] = {primary_name: oracle_parity(ctx)}
        if second is not None:
            result["oracle_parity"]["mtp"] = oracle_parity(ctx2)
        eprint(f"oracle parity {result['oracle_parity']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
