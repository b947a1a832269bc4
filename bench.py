"""Throughput of the paged-KV hot path on one MI355X, as one JSON line.

Default run: all five workloads of the path, one after another, reported in one line.
* ``long_decode`` (the headline, top level): 7B-shaped decode, batch 64, contexts U[4096, 8192],
  32 query / 8 KV heads, head_dim 128, bf16 KV;
* nested under ``configs`` with the same fields: ``tiny_fp32`` (4 sequences, contexts
  {1, 255, 256, 600}, fp32), ``qwen3_decode`` (batch 256, contexts U[100, 2048], 16/8 heads, bf16),
  ``prefill_prefix`` (32 prompts sharing 512-token prefixes in groups of 8, chunks of at most 4096
  new tokens, 16/8 heads, bf16) and ``int8_decode`` (batch 128, contexts U[512, 8192], 32/32 heads,
  int8 KV with per-(block, head) scales), plus ``long_decode`` itself.

A decode *step* is everything a decode iteration does on the path: the block manager appends one
token per sequence (host C++), block tables, lengths and slots go to the device in one pinned copy,
kv_store writes the new K/V rows, and the decode kernels attend over the whole paged context, so
contexts grow by one token per step as in a real decode loop.  A prefill step is the whole chunked
workload: every chunk's store and prefill attention.  All inputs are seeded synthetic data and are
resident in HBM before timing starts.

``--config NAME`` runs one workload alone (also ``beam_decode``, ``beam_long``, ``prefill_long``, ``int8_store``).

Reported per workload:
* ``value`` / ``ms_per_step`` -- whole steps timed by the wall clock (K steps after W warm-up steps);
* ``roofline`` -- the dominant kernel's algorithmic traffic (decode: KV bytes of the valid tokens;
  prefill: causal flops) divided by its average duration, timed with HIP events on the launch
  stream in a second pass of K steps, each preceded by a 512 MiB write that evicts L2 and the
  MALL (``--flush-mb``), against MI355X's published peak (8 TB/s HBM3E; 2.5 PFLOP/s dense bf16);
* ``cpu_baseline`` -- the fp64 oracle on a bounded sample of the same workload, split over
  worker processes on the host's cores (one thread each), timed before the GPU is touched.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--seed S]
"""

import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
DEFAULT_STEPS, DEFAULT_WARMUP = 20, 3
BF16_PEAK_TFLOPS = 2516.6  # dense MFMA, 256 CUs at 2.4 GHz


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=DEFAULT_STEPS)
    ap.add_argument("--warmup", type=int, default=DEFAULT_WARMUP)
    ap.add_argument("--config", default=None, help="one workload alone (default: every workload of the path)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--max-splits", type=int, default=0)
    ap.add_argument("--window", type=int, default=0,
                    help="sliding-window attention: each query attends its last W keys (0: every key)")
    ap.add_argument("--fused", action="store_true",
                    help="decode: store the new tokens inside the attention launch (pkv_decode_store_attend)")
    ap.add_argument("--unsplit", action="store_true",
                    help="prefill: keep every work item whole (no key-range split of launches that leave CUs idle)")
    ap.add_argument("--ungrouped", action="store_true",
                    help="beam workloads: attend every beam on its own (pkv_paged_attn_decode); by default a "
                         "step whose requests share at least runner.GROUP_MIN_SHARED keys on average reads "
                         "each request's shared blocks once (pkv_paged_attn_decode_grouped)")
    ap.add_argument("--group-splits", type=int, default=0,
                    help="beam configs: cut each request's shared keys into up to this many splits "
                         "(pkv_paged_attn_decode_grouped_split; 1: one workgroup per request and KV head; "
                         "0: the runner's choice, about one workgroup per CU)")
    ap.add_argument("--requests", type=int, default=0,
                    help="beam configs: this many requests instead of the workload's (few requests: few "
                         "groups, where --group-splits matters)")
    ap.add_argument("--grouped", action="store_true",
                    help="beam workloads: always read each request's shared blocks once")
    ap.add_argument("--graph", action="store_true",
                    help="decode: replay each step's upload, store and attention from HIP graphs")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="write this many MiB of scratch before every step of the event pass, so the timed "
                         "kernels read a cold L2 and MALL (0: no flush); the wall-clock pass never flushes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="CPU time (summed over the worker processes) the oracle baseline may spend per workload")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain 1 GiB device copy (to scale hardware byte counters) and exit")
    ap.add_argument("--summarize", metavar="NAME",
                    help="write profiles/NAME.txt from rocprofv3 CSV output (see --prof-dir) and exit")
    ap.add_argument("--prof-dir", default="gpurun_out/prof")
    ap.add_argument("--prof-cmd", default="", help="the command lines that produced the CSVs (recorded)")
    ap.add_argument("--prof-workload", default=None, help="the workload whose counters the CSVs hold")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)



# ------------------------------------------------------------------------------------ profiles
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = {"decode_split_kernel": "decode.hip", "decode_group_kernel": "decode.hip", "prefill_kernel": "prefill.hip",
                  "prefill_merge_kernel": "prefill.hip", "kv_store_kernel": "kv_store.hip", "kv_store_quant_kernel": "kv_store.hip"}


def source_hash(kernel):
    """Short hash of the HIP source a kernel is built from (ties a stored counter reading to a kernel version)."""
    import hashlib
    src = os.path.join(ROOT, "paged_kv_cache_kvcache_amd", "csrc", KERNEL_SOURCES[kernel])
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def summarize(name, prof_dir, cmd, workload=None):
    """Summarise rocprofv3 CSVs: kernel stats, and FETCH_SIZE / WRITE_SIZE per dispatch scaled by the
    same counters' reading for a plain copy of known size."""
    import csv
    import glob
    out = [f"# {name}", f"# produced by: {cmd}", ""]
    for f in sorted(glob.glob(os.path.join(prof_dir, "*kernel_stats.csv"))):
        out.append(f"## kernel stats ({os.path.basename(f)})")
        out.append("kernel | calls | avg us | min us | max us | share %")
        for r in csv.DictReader(open(f)):
            out.append(f"{r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                       f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}")
        out.append("")
    counters = {}
    for f in sorted(glob.glob(os.path.join(prof_dir, "*counter_collection.csv"))):
        for r in csv.DictReader(open(f)):
            key = (os.path.basename(f).split("_")[0], r["Kernel_Name"], r["Counter_Name"])
            counters.setdefault(key, []).append(float(r["Counter_Value"]))
    if counters:
        out.append("## hardware counters (per dispatch, KiB for *_SIZE)")
        scale = {}
        for (run, kern, ctr), v in sorted(counters.items()):
            avg = sum(v) / len(v)
            if ctr.startswith(("SQ_", "GRBM_")) and "prefill_kernel" not in kern:
                continue  # shader-sequencer passes are taken for the prefill kernel
            out.append(f"{run} | {kern[:80]} | {ctr} | n={len(v)} | avg={avg:.6g} | min={min(v):.6g} | max={max(v):.6g}")
            if run == "copy" and "copyBuffer" in kern:
                scale[ctr] = (1 << 30) / (avg * 1024)
        out.append("")
        if scale:
            out.append("copy calibration (bytes of a 1 GiB copy / counter bytes): " +
                       ", ".join(f"{k} x{v:.4f}" for k, v in sorted(scale.items())))
        # derived shader-sequencer figures (counters are summed over the 8 XCDs; GRBM_GUI_ACTIVE
        # counts each XCD's busy cycles, the SQ cycle counters each SIMD's or each wave's)
        for kern in ("prefill_kernel",):
            avg = {c: sum(v) / len(v) for (run, k, c), v in counters.items() if kern in k and c.startswith(("SQ_", "GRBM_"))}
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
                simd_cycles = avg["GRBM_GUI_ACTIVE"] / 8 * 1024  # 1024 SIMDs busy for the kernel's cycles
                out.append(f"DERIVED {kern}: MFMA busy {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.3f} of SIMD cycles "
                           f"(SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024))")
                if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
                    out.append(f"DERIVED {kern}: VALU co-issued during {avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / avg['SQ_VALU_MFMA_BUSY_CYCLES']:.3f}"
                               f" of MFMA-busy cycles")
                for c in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY"):
                    if c in avg and "SQ_WAVE_CYCLES" in avg:
                        out.append(f"DERIVED {kern}: {c} {avg[c] / avg['SQ_WAVE_CYCLES']:.3f} of wave cycles")
            if "SQ_INSTS_MFMA" in avg and "SQ_INSTS_VALU" in avg:
                out.append(f"DERIVED {kern}: {avg['SQ_INSTS_VALU'] / avg['SQ_INSTS_MFMA']:.2f} VALU and "
                           f"{avg.get('SQ_INSTS_LDS', 0) / avg['SQ_INSTS_MFMA']:.2f} LDS instructions per MFMA; "
                           f"LDS bank conflicts {avg.get('SQ_LDS_BANK_CONFLICT', 0):.0f}")
        for kern in ("decode_split_kernel", "decode_group_kernel", "prefill_kernel", "prefill_merge_kernel",
                     "kv_store_quant_kernel"):
            f = [sum(v) / len(v) for (run, k, c), v in counters.items() if kern in k and c == "FETCH_SIZE"]
            w = [sum(v) / len(v) for (run, k, c), v in counters.items() if kern in k and c == "WRITE_SIZE"]
            if f and w and "FETCH_SIZE" in scale and "WRITE_SIZE" in scale:
                fb = f[0] * 1024 * scale["FETCH_SIZE"]
                wb = w[0] * 1024 * scale["WRITE_SIZE"]
                out.append(f"TRAFFIC {kern} workload={workload or name} source={source_hash(kern)} "
                           f"fetch_bytes={fb:.6g} write_bytes={wb:.6g} total_bytes={fb + wb:.6g}")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    path = os.path.join(ROOT, "profiles", name + ".txt")
    open(path, "w").write("\n".join(out) + "\n")
    print(path)


def stored_traffic(kernel, workload, nch=1):
    """HBM bytes of one step (counter bytes per dispatch x ``nch`` dispatches) from a committed
    counter summary of this workload, if taken on the current kernel source."""
    import glob
    h = source_hash(kernel)
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        for line in open(f):
            if line.startswith(f"TRAFFIC {kernel} workload={workload} source={h} "):
                return float(line.split("total_bytes=")[1].split()[0]) * nch
    return None

# ------------------------------------------------------------------------------------ decode
def decode_max_context(lens, warmup, steps):
    """The context capacity a decode line plans for: its warm-up, wall-clock and event passes each
    append one token per step."""
    return max(lens) + warmup + 2 * steps


def bench_decode(args, cfg, wl=None, cpu=None):
    """One decode workload on the GPU; ``wl`` (generated here when None) and ``cpu`` (the oracle
    baseline, timed here before the GPU is touched when None and not disabled)."""
    import torch
    import workloads as W
    from paged_kv_cache_kvcache_amd import BF16, F32, I8, decode_plan
    from paged_kv_cache_kvcache_amd import runner as R

    dev = torch.device("cuda:0")
    dtype = cfg["dtype"]
    kvdt = {"f32": F32, "bf16": BF16, "i8": I8}[dtype]
    B, Hq, Hkv, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    # warm-up, K steps timed by the wall clock (the throughput), then K steps with HIP events around
    # the attention launch (its duration); the events cost the stream several microseconds per step,
    # so they stay out of the throughput pass
    nsteps = args.warmup + 2 * args.steps
    t0 = time.time()
    if wl is None:
        wl = W.decode_workload(cfg, args.seed)
    if cpu is None and not args.no_cpu_baseline:
        cpu = cpu_baseline_decode(wl, args.window, args.cpu_seconds)
    lens = wl["lens"]
    # the pool also holds the tokens the timed steps append
    nb = max(wl["num_blocks"], W.pool_blocks(cfg, [L + nsteps for L in lens]))
    order = W.free_order(cfg, args.seed, nb)
    log(f"[bench] generated {cfg['name']} (B={B}, sum ctx={sum(lens)}) in {time.time() - t0:.1f}s")

    kv = R.PagedKV(nb, Hkv, D, kvdt, order, device=dev)
    ids = list(range(B))
    if dtype == "i8":
        parts = [(s["kq"], s["vq"], s["k_tok_scale"], s["v_tok_scale"]) for s in wl["seqs"]]
    else:
        parts = [(s["k"], s["v"], None, None) for s in wl["seqs"]]
    # history = every token but the last; the workload's own new token is the first timed append
    R.admit_and_store(kv, ids, [s["tokens"][:-1] for s in wl["seqs"]], [p[0][:-1] for p in parts],
                      [p[1][:-1] for p in parts],
                      [None if p[2] is None else p[2][:-1] for p in parts],
                      [None if p[3] is None else p[3][:-1] for p in parts])
    max_ctx = decode_max_context(lens, args.warmup, args.steps)
    if (args.graph or args.fused) and args.window:
        raise SystemExit("--graph and --fused have no sliding window")
    batch = R.DecodeBatch(kv, Hq, ids, max_ctx, args.max_splits, window=args.window)
    # the plan the kernel uses: a window of W keys spans at most ceil((W + 255) / 256) blocks
    span = min(max_ctx, args.window + 255) if args.window > 0 else max_ctx
    splits, bps = decode_plan(B, Hkv, span, args.max_splits)

    # per-step inputs, resident on the device before timing
    steps = []
    blk_scale = {}
    cur = list(lens)
    for s in range(nsteps):
        if s == 0:
            tokens = np.array([x["tokens"][-1] for x in wl["seqs"]], dtype=np.int32)
            q = np.stack([x["q"] for x in wl["seqs"]])
            k = np.stack([p[0][-1] for p in parts])
            v = np.stack([p[1][-1] for p in parts])
            ks = vs = None
            if dtype == "i8":
                ks = np.stack([p[2][-1] for p in parts])
                vs = np.stack([p[3][-1] for p in parts])
                for b, x in enumerate(wl["seqs"]):
                    blk_scale[b] = (x["k_blk_scale"][-1].copy(), x["v_blk_scale"][-1].copy())
        else:
            inp = W.decode_step_inputs(cfg, args.seed, s, B)
            tokens, q, k, v = inp["tokens"], inp["q"], inp["k"], inp["v"]
            ks = vs = None
            if dtype == "i8":
                bk = np.stack([np.full(Hkv, np.nan, np.float32) if (cur[b] - 1) % 256 == 0 else blk_scale[b][0]
                               for b in range(B)])
                bv = np.stack([np.full(Hkv, np.nan, np.float32) if (cur[b] - 1) % 256 == 0 else blk_scale[b][1]
                               for b in range(B)])
                k, ks = W.int8_encode_token(W.bf16_bits_to_f32(k), bk)
                v, vs = W.int8_encode_token(W.bf16_bits_to_f32(v), bv)
                for b in range(B):
                    blk_scale[b] = (ks[b].copy(), vs[b].copy())
        dv = lambda a: None if a is None else (R.bf16_tensor(a, dev) if a.dtype == np.uint16 else
                                               torch.from_numpy(np.ascontiguousarray(a)).to(dev))
        steps.append(dict(tokens=tokens, q=dv(q), k=dv(k), v=dv(v), ks=dv(ks), vs=dv(vs), ctx=list(cur)))
        cur = [c + 1 for c in cur]
    out = torch.empty((B, Hq, D), dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device=dev)
    scale = 1.0 / math.sqrt(D)
    esize = {"f32": 4, "bf16": 2, "i8": 1}[dtype]

    def kv_bytes(ctx):
        # the keys attended: the whole context, or the last `window` of it
        ctx = [min(c, args.window) if args.window > 0 else c for c in ctx]
        b = sum(ctx) * Hkv * D * esize * 2
        if dtype == "i8":
            b += sum(-(-c // 256) for c in ctx) * Hkv * 2 * 4
        return b

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    flush = torch.empty(args.flush_mb << 20, dtype=torch.uint8, device=dev) if args.flush_mb > 0 else None

    def run(i, timed_idx=None):
        st = steps[i]
        if flush is not None and timed_idx is not None:  # the event pass reads a cold cache
            flush.fill_(i & 0xFF)
        slots = kv.alloc.append_batch(batch.ids, st["tokens"])
        batch.upload_step_metadata(slots)
        if args.fused:
            if timed_idx is not None:
                ev[timed_idx][0].record(stream)
            batch.store_attend(st["q"], st["k"], st["v"], scale, out, st["ks"], st["vs"])
        else:
            kv.store(batch.slots, st["k"], st["v"], st["ks"], st["vs"])
            if timed_idx is not None:
                ev[timed_idx][0].record(stream)
            batch.attend(st["q"], scale, out)
        if timed_idx is not None:
            ev[timed_idx][1].record(stream)

    if args.graph:
        # the step's inputs arrive in the graphs' fixed buffers with one device copy (as if the
        # projections had written them there); upload, store and attention replay from graphs
        gb = R.GraphedDecodeBatch(kv, Hq, ids, max_ctx, scale, args.max_splits)
        for st in steps:
            st["blob"] = gb.pack_inputs(*[st[x] for x in ("q", "k", "v", "ks", "vs") if st[x] is not None])

        def run(i, timed_idx=None):  # noqa: F811
            st = steps[i]
            if flush is not None and timed_idx is not None:
                flush.fill_(i & 0xFF)
            gb.inputs.copy_(st["blob"])
            gb.step(st["tokens"], None if timed_idx is None else ev[timed_idx])

    # Python's cyclic GC can pause the host for tens of ms inside a step; like timeit (and serving
    # loops), collect once and keep it off while timing
    gc.collect()
    gc.disable()
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        run(args.warmup + j)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ev_steps = [args.warmup + args.steps + j for j in range(args.steps)]
    for j, i in enumerate(ev_steps):
        run(i, j)
    torch.cuda.synchronize()
    gc.enable()
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    avg_kern_s = sum(kern_ms) / len(kern_ms) / 1e3
    bytes_per_launch = sum(kv_bytes(steps[i]["ctx"]) for i in ev_steps) / args.steps
    achieved = bytes_per_launch / avg_kern_s / 1e9
    log(f"[bench] splits={splits} blocks/split={bps}; decode kernel avg {avg_kern_s * 1e6:.1f} us, "
        f"{achieved:.0f} GB/s; step {elapsed / args.steps * 1e3:.3f} ms")

    res = dict(
        metric="paged decode tokens/s + KV HBM GB/s (% of peak); prefill TFLOP/s",
        value=B * args.steps / elapsed, unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=elapsed / args.steps * 1e3, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype=dtype, data="synthetic",
        config=dict(workload=cfg["name"], batch=B, context=f"U[{cfg['ctx'][0]}, {cfg['ctx'][1]}]" if isinstance(
            cfg["ctx"], tuple) else str(cfg["ctx"]), q_heads=Hq, kv_heads=Hkv, head_dim=D, block_size=256,
            splits=splits, blocks_per_split=bps, window=args.window, hip_graph=bool(args.graph),
            flush_mb=args.flush_mb, fused_store=bool(args.fused), seed=args.seed),
        decode_kernel_us=avg_kern_s * 1e6, decode_tokens_per_s_kernel=B / avg_kern_s,
        kv_gbs=achieved,
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s", frac=achieved / HBM_PEAK_GBS,
                      traffic=stored_traffic("decode_split_kernel", cfg["name"], nch=1)
                      if args.seed == 0 and args.window == 0 and not args.graph and not args.fused and
                      args.max_splits == 0 else None,
                      kernel="decode (split kernel + LSE reduce when splits > 1)",
                      bytes_per_launch=bytes_per_launch, cold_cache=args.flush_mb > 0),
    )
    if cpu is not None:
        res["cpu_baseline"] = cpu
    return res


# ------------------------------------------------------------------------- oracle baselines
# The oracle, as it stands, on a bounded sample of the workload.  Its items (sequences, prompts,
# rows, repetitions) are independent, so the sample is cut into contiguous slices that worker
# processes run at once, one thread each, over the host cores this process may use (at most 16,
# one GPU's share of the host).  The pool is forked before the GPU is touched, and the workload it
# reads is shared with the parent, not copied.
_ORACLE_JOBS = {}


def host_workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _oracle_noop(_):
    return os.getpid()


def _oracle_slice(task):
    name, lo, hi = task
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        t0 = time.perf_counter()
        units = _ORACLE_JOBS[name](lo, hi)
        return units, time.perf_counter() - t0


def parallel_oracle(fn, total, cpu_seconds=20.0):
    """Run ``fn(lo, hi)`` (the oracle on items lo..hi-1, returning the units of work it did) over a
    sample of the first n items, n sized from one item alone so that the workers spend about
    ``cpu_seconds`` in total.  Returns (units, wall seconds, workers, CPU seconds, n)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        t0 = time.perf_counter()
        fn(0, 1)  # calibration: one item alone
        one = max(time.perf_counter() - t0, 1e-4)
    workers = host_workers()
    n = int(min(total, max(1, cpu_seconds / one)))
    w = min(workers, n)
    bounds = [n * i // w for i in range(w + 1)]
    key = f"job{len(_ORACLE_JOBS)}"
    _ORACLE_JOBS[key] = fn
    with ProcessPoolExecutor(max_workers=w, mp_context=mp.get_context("fork")) as ex:
        list(ex.map(_oracle_noop, range(w)))  # every worker is up before the clock starts
        t0 = time.perf_counter()
        res = list(ex.map(_oracle_slice, [(key, bounds[i], bounds[i + 1]) for i in range(w)]))
        wall = time.perf_counter() - t0
    del _ORACLE_JOBS[key]
    return sum(r[0] for r in res), wall, w, sum(r[1] for r in res), n


def _pool_note(w, cpu_s, wall):
    return f"{w} worker processes, one thread each: {cpu_s:.1f} s of CPU in {wall:.2f} s"


def cpu_baseline_decode(wl, window=0, cpu_seconds=20.0):
    """The oracle's whole decode step (its block manager, store and attention) on a sample of the
    sequences, in slices."""
    import workloads as W
    from oracle.steps import decode_step

    def run(lo, hi):
        sub = dict(wl)
        sub["lens"] = wl["lens"][lo:hi]
        sub["seqs"] = wl["seqs"][lo:hi]
        sub["num_blocks"] = W.pool_blocks(wl["cfg"], sub["lens"])
        sub["free_order"] = W.free_order(wl["cfg"], wl["seed"], sub["num_blocks"])
        decode_step(sub, window)
        return hi - lo

    units, wall, w, cpu_s, n = parallel_oracle(run, len(wl["lens"]), cpu_seconds)
    win = f" over the last {window} keys" if window > 0 else ""
    return dict(value=units / wall, unit="tokens/s", cores=w, kind="oracle",
                sample=f"first {n} of {len(wl['lens'])} sequences ({sum(wl['lens'][:n])} context tokens), one decode "
                       f"step: oracle block manager + store + fp64 attention{win}; {_pool_note(w, cpu_s, wall)}")


# ------------------------------------------------------------------------------------ prefill
def bench_prefill(args, cfg, wl=None, cpu=None):
    """The chunked prefill workload on the GPU (``wl``, ``cpu`` as in :func:`bench_decode`)."""
    import torch
    import workloads as W
    from paged_kv_cache_kvcache_amd import (BF16, desc_of, kv_store, paged_attn_prefill_split, prefill_split_order,
                                            prefill_split_workspace_bytes, prefill_work_order)
    from paged_kv_cache_kvcache_amd import runner as R

    dev = torch.device("cuda:0")
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    if wl is None:
        wl = W.prefill_workload(cfg, args.seed)
    if cpu is None and not args.no_cpu_baseline and args.window == 0:
        cpu = (cpu_baseline_prefill_rows(wl, args.cpu_seconds) if cfg.get("split") else
               cpu_baseline_prefill(wl, args.cpu_seconds))
    prompts = wl["prompts"]
    kv = R.PagedKV(wl["num_blocks"], Hkv, D, BF16, wl["free_order"], device=dev)
    t0 = time.perf_counter()
    ncached = [kv.alloc.add_seq(i, p["tokens"]) for i, p in enumerate(prompts)]
    n_new = [len(p["tokens"]) - c for p, c in zip(prompts, ncached)]
    # chunks as segments (prompt, start, end) of the prompts' new tokens: whole prompts, or prompts
    # split across chunks when the workload asks for it
    chunks = (W.pack_chunks_split(n_new, cfg["chunk"]) if cfg.get("split") else
              [[(i, 0, n_new[i]) for i in ch] for ch in W.pack_chunks(n_new, cfg["chunk"])])
    metas = []
    for ch in chunks:
        ids = [i for i, _, _ in ch]
        cu, lk, slots = kv.alloc.prefill_segment_slots(ids, [a for _, a, _ in ch], [b for _, _, b in ch],
                                                       sum(b - a for _, a, b in ch))
        tab, lens = kv.alloc.block_tables(ids, wl["num_blocks"])  # whole sequences, later segments included
        mb = max(1, -(-int(lens.max()) // 256))
        tab = np.ascontiguousarray(tab[:, :mb])
        # the chunk's work items, heaviest first in CU-balanced rounds, long ones cut into key-range
        # pieces when the launch would leave CUs idle (pkv_prefill_split_order)
        split = prefill_split_order(desc_of(kv.k_cache), Hq, cu, lk, True, args.window)
        if args.unsplit:  # the same work order with every item whole
            items, rows = prefill_work_order(desc_of(kv.k_cache), Hq, cu, lk, True, args.window)
            whole = np.stack([items, np.zeros_like(items), np.full_like(items, 2**31 - 1), np.full_like(items, -1)], 1)
            split = (whole, np.zeros((0, 4), np.int32), 0, rows)
        metas.append((cu, lk, slots, tab, mb, split))
    host_s = time.perf_counter() - t0
    # device-resident inputs of every chunk
    dchunks, flops = [], 0
    ws_bytes = max(prefill_split_workspace_bytes(desc_of(kv.k_cache), Hq, m[5][2], m[5][3]) for m in metas)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes > 0 else None
    for ch, (cu, lk, slots, tab, mb, split) in zip(chunks, metas):
        dv = lambda key: R.bf16_tensor(np.concatenate([prompts[i][key][ncached[i] + a:ncached[i] + b]
                                                       for i, a, b in ch]), dev)
        q, k, v = dv("q"), dv("k"), dv("v")
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        dchunks.append(dict(q=q, k=k, v=v, cu=to(cu), lk=to(lk), slots=to(slots), tab=to(tab).view(len(ch), mb),
                            pieces=to(split[0]), merges=to(split[1]), n_slots=split[2], tile_rows=split[3],
                            max_q=int(np.diff(cu).max()), max_k=int(lk.max()),
                            out=torch.empty_like(q)))
        for b in range(len(ch)):
            nq, L = int(cu[b + 1] - cu[b]), int(lk[b])
            # causal pairs (within the window when there is one)
            flops += 4 * D * Hq * sum(min(L - nq + i + 1, args.window) if args.window > 0 else L - nq + i + 1
                                      for i in range(nq))
    scale = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream()
    nch = len(dchunks)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nch)]
          for _ in range(args.steps)]

    flush = torch.empty(args.flush_mb << 20, dtype=torch.uint8, device=dev) if args.flush_mb > 0 else None

    def run(timed=None):
        if flush is not None and timed is not None:  # the event pass starts each step on a cold cache
            flush.fill_(timed & 0xFF)
        for c, d in enumerate(dchunks):
            kv_store(d["k"], d["v"], d["slots"], kv.k_cache, kv.v_cache)
            if timed is not None:
                ev[timed][c][0].record(stream)
            paged_attn_prefill_split(d["q"], d["cu"], d["lk"], d["max_q"], d["max_k"], kv.k_cache, kv.v_cache,
                                     d["tab"], scale, d["pieces"], d["merges"], d["n_slots"], d["tile_rows"],
                                     workspace, True, args.window, out=d["out"])
            if timed is not None:
                ev[timed][c][1].record(stream)

    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    # K steps timed by the wall clock (the throughput), then K steps with events around each chunk's
    # attention launch (their durations), as in the decode line
    t0 = time.perf_counter()
    for j in range(args.steps):
        run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for j in range(args.steps):
        run(j)
    torch.cuda.synchronize()
    gc.enable()
    kern_s = sum(a.elapsed_time(b) for row in ev for a, b in row) / args.steps / 1e3
    tflops = flops / kern_s / 1e12
    total_new = sum(n_new)
    log(f"[bench] prefill {nch} chunks, {total_new} new tokens, {flops / 1e9:.2f} GFLOP; prefill kernels "
        f"{kern_s * 1e6:.1f} us/step -> {tflops:.1f} TFLOP/s; step {elapsed / args.steps * 1e3:.3f} ms")
    # counter traffic of one step (mean per dispatch x dispatches: one attention launch per chunk,
    # one merge per chunk with split items), when taken on this workload and the current source
    traffic = None
    if args.seed == 0 and args.window == 0:
        n_merge = sum(1 for d in dchunks if d["n_slots"] > 0)
        traffic = stored_traffic("prefill_kernel", cfg["name"], nch)
        if traffic is not None and n_merge:
            merge = stored_traffic("prefill_merge_kernel", cfg["name"], n_merge)
            traffic = None if merge is None else traffic + merge
    res = dict(
        metric="paged decode tokens/s + KV HBM GB/s (% of peak); prefill TFLOP/s",
        value=total_new * args.steps / elapsed, unit="prefill tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=elapsed / args.steps * 1e3, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload=cfg["name"], prompts=cfg["B"], prompt_len=f"U[{cfg['ctx'][0]}, {cfg['ctx'][1]}]",
                    shared_prefix=cfg["shared"], group=cfg["group"], chunk_tokens=cfg["chunk"], window=args.window,
                    q_heads=Hq,
                    kv_heads=Hkv, head_dim=D, block_size=256, chunks=nch, new_tokens=total_new,
                    cached_tokens=sum(ncached), split_underfilled=not args.unsplit, seed=args.seed),
        prefill_kernel_us=kern_s * 1e6, prefill_tflops=tflops, host_admit_us=host_s * 1e6,
        roofline=dict(bound="mfma", achieved=tflops, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                      frac=tflops / BF16_PEAK_TFLOPS, traffic=traffic, kernel="prefill (all chunks of one step)",
                      flops_per_step=flops, cold_cache=args.flush_mb > 0),
    )
    if cpu is not None:
        res["cpu_baseline"] = cpu
    return res


# ------------------------------------------------------------------------- int8 quantising store
def bench_int8_store(args, cfg):
    """The prefill workload's new K/V rows (bf16) written by the quantising store into int8 caches:
    one step = every chunk's store, in chunk order."""
    import torch
    import workloads as W
    from paged_kv_cache_kvcache_amd import I8, store_runs
    from paged_kv_cache_kvcache_amd import runner as R

    dev = torch.device("cuda:0")
    Hkv, D = cfg["Hkv"], cfg["D"]
    wl = W.prefill_workload(cfg, args.seed)
    cpu = None if args.no_cpu_baseline else cpu_baseline_int8_store(wl, args.cpu_seconds)
    prompts = wl["prompts"]
    kv = R.PagedKV(wl["num_blocks"], Hkv, D, I8, wl["free_order"], device=dev)
    ncached = [kv.alloc.add_seq(i, p["tokens"]) for i, p in enumerate(prompts)]
    n_new = [len(p["tokens"]) - c for p, c in zip(prompts, ncached)]
    chunks = W.pack_chunks(n_new, cfg["chunk"])
    dchunks, blocks = [], 0
    for ch in chunks:
        _, _, slots = kv.alloc.prefill_slots(ch, sum(n_new[i] for i in ch))
        runs, n_runs, longest = store_runs(slots)
        dv = lambda key: R.bf16_tensor(np.concatenate([prompts[i][key][ncached[i]:] for i in ch]), dev)
        dchunks.append(dict(k=dv("k"), v=dv("v"), slots=torch.from_numpy(np.ascontiguousarray(slots)).to(dev),
                            runs=(torch.from_numpy(runs).to(dev), n_runs, longest)))
        blocks += n_runs
    total_new = sum(n_new)
    # algorithmic bytes per step: bf16 rows read, int8 codes written, one fp32 scale per (block, head)
    # written, for K and V
    step_bytes = 2 * (total_new * Hkv * D * (2 + 1) + blocks * Hkv * 4)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def run(j=None):
        if j is not None:
            ev[j][0].record(stream)
        for d in dchunks:
            kv.store_quant(d["slots"], d["k"], d["v"], d["runs"])
        if j is not None:
            ev[j][1].record(stream)

    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for j in range(args.steps):  # the event pass: store durations, kept out of the wall clock
        run(j)
    torch.cuda.synchronize()
    gc.enable()
    kern_s = sum(a.elapsed_time(b) for a, b in ev) / args.steps / 1e3
    gbs = step_bytes / kern_s / 1e9
    # counter traffic per dispatch (mean over the chunks), when taken on the current kernel source
    traffic = stored_traffic("kv_store_quant_kernel", cfg["name"], len(dchunks)) if args.seed == 0 else None
    log(f"[bench] int8 store: {len(dchunks)} chunks, {total_new} new tokens, {step_bytes / 1e6:.1f} MB; "
        f"{kern_s * 1e6:.1f} us/step -> {gbs:.0f} GB/s")
    return dict(
        metric="int8 quantising store: stored tokens/s + HBM GB/s (% of peak)",
        value=total_new * args.steps / elapsed, unit="stored tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=elapsed / args.steps * 1e3, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16->i8", data="synthetic",
        config=dict(workload=cfg["name"], prompts=cfg["B"], new_tokens=total_new, kv_heads=Hkv, head_dim=D,
                    block_size=256, chunks=len(dchunks), seed=args.seed),
        store_kernel_us=kern_s * 1e6,
        roofline=dict(bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=gbs / HBM_PEAK_GBS,
                      traffic=traffic, kernel="kv_store_quant (all chunks of one step)", bytes_per_step=step_bytes),
        cpu_baseline=cpu,
    )


def cpu_baseline_int8_store(wl, cpu_seconds=20.0):
    """The oracle's quantising store of the first chunk's new rows (slots from the oracle's own block
    manager), repeated; each repetition is one item."""
    import workloads as W
    from oracle import allocator as OA
    from oracle import attention as OT
    cfg = wl["cfg"]
    Hkv, D, prompts = cfg["Hkv"], cfg["D"], wl["prompts"]
    a = OA.Allocator(wl["num_blocks"], wl["free_order"])
    ncached = [a.add_seq(i, p["tokens"]) for i, p in enumerate(prompts)]
    first = W.pack_chunks([len(p["tokens"]) - c for p, c in zip(prompts, ncached)], cfg["chunk"])[0]
    _, _, slots = a.prefill_slots(first)
    k = W.bf16_bits_to_f32(np.concatenate([prompts[i]["k"][ncached[i]:] for i in first]))
    v = W.bf16_bits_to_f32(np.concatenate([prompts[i]["v"][ncached[i]:] for i in first]))
    kc = np.zeros((wl["num_blocks"], Hkv, 256, D), np.int8)
    ks = np.zeros((wl["num_blocks"], Hkv), np.float32)

    def run(lo, hi):
        for _ in range(lo, hi):
            OT.kv_store_quant(kc, kc, ks, ks, k, v, slots)
        return (hi - lo) * len(slots)

    units, wall, w, cpu_s, n = parallel_oracle(run, 1 << 20, cpu_seconds)
    return dict(value=units / wall, unit="stored tokens/s", cores=w, kind="oracle",
                sample=f"the first chunk's {len(slots)} new tokens (K and V, {Hkv} heads) stored {n} times: oracle "
                       f"quantising store; {_pool_note(w, cpu_s, wall)}")


def bench_beam(args, cfg):
    """Beam search over decode prompts: every step each request's new beams fork from seeded parents
    among its current beams (ocdem.com nano-vllm article, §2.1: the sequences of a request share
    blocks), the old beams end, one token is appended per beam with copy-on-write (all but the last
    appender into a shared partial block copy its rows in use), then the store and the attention
    over every beam."""
    import torch
    import workloads as W
    from paged_kv_cache_kvcache_amd import BF16
    from paged_kv_cache_kvcache_amd import runner as R

    dev = torch.device("cuda:0")
    NR, NBM, Hq, Hkv, D = cfg["B"], cfg["beams"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    B = NR * NBM
    nsteps = args.warmup + 2 * args.steps  # warm-up, the wall-clock pass, the event pass
    wl = W.decode_workload(cfg, args.seed)
    cpu = None if args.no_cpu_baseline else cpu_baseline_beam(wl, args.seed, args.cpu_seconds)
    lens = wl["lens"]
    # prompts, plus per beam a private partial block and the blocks its appends open
    nb = W.pool_blocks(cfg, lens) + B * (2 + -(-nsteps // 256))
    kv = R.PagedKV(nb, Hkv, D, BF16, W.free_order(cfg, args.seed, nb), device=dev)
    R.admit_and_store(kv, list(range(NR)), [s["tokens"] for s in wl["seqs"]], [s["k"] for s in wl["seqs"]],
                      [s["v"] for s in wl["seqs"]])
    max_ctx = max(lens) + nsteps
    # the beams of a request are consecutive: grouped attention reads their shared blocks once
    batch = R.DecodeBatch(kv, Hq, list(range(B)), max_ctx, args.max_splits, cow=True,
                          group_size=0 if args.ungrouped else NBM,
                          group_min_shared=0 if args.grouped else R.GROUP_MIN_SHARED,
                          group_splits=args.group_splits)
    steps = []
    for s in range(nsteps):
        inp = W.decode_step_inputs(cfg, args.seed, s, B)
        steps.append(dict(tokens=inp["tokens"], parents=W.beam_parents(cfg, args.seed, s),
                          q=R.bf16_tensor(inp["q"], dev), k=R.bf16_tensor(inp["k"], dev),
                          v=R.bf16_tensor(inp["v"], dev)))
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    scale = 1.0 / math.sqrt(D)
    row_bytes = Hkv * D * 2
    stream = torch.cuda.current_stream()
    mk = lambda: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
    ev_copy, ev_dec = mk(), mk()
    state = dict(beams=np.arange(NR, dtype=np.int64)[:, None], next_id=NR)  # [request][beam] ids
    log_rows, log_copies, log_tables, log_grouped = [], [], [], []

    def unique_rows(tab, lens):
        """Rows of the distinct physical blocks the step's beams attend (each block read once)."""
        used = {}
        for row, L in zip(tab, lens):
            for j in range(-(-int(L) // 256)):
                b = int(row[j])
                used[b] = max(used.get(b, 0), min(256, int(L) - 256 * j))
        return sum(used.values())

    def run(i, timed_idx=None):
        st = steps[i]
        alloc = kv.alloc
        nid = state["next_id"]
        cur = state["beams"]
        par = np.take_along_axis(cur, st["parents"] % cur.shape[1], axis=1).ravel()
        new = np.arange(nid, nid + B, dtype=np.int64)
        alloc.fork_batch(par, new)
        alloc.free_batch(cur.ravel())
        state["beams"] = new.reshape(NR, NBM)
        state["next_id"] = nid + B
        slots, src, dst, rows = alloc.append_batch_cow(new, st["tokens"])
        batch.set_sequences(new)
        batch.upload_step_metadata(slots, (src, dst, rows))
        if timed_idx is not None:
            ev_copy[timed_idx][0].record(stream)
        batch.copy_on_write()
        if timed_idx is not None:
            ev_copy[timed_idx][1].record(stream)
        kv.store(batch.slots, st["k"], st["v"])
        if timed_idx is not None:
            ev_dec[timed_idx][0].record(stream)
        batch.attend(st["q"], scale, out)
        if timed_idx is not None:
            ev_dec[timed_idx][1].record(stream)
            log_grouped.append(batch.grouped)
            log_rows.append(int(rows.sum()))
            log_copies.append(len(src))
            log_tables.append((batch.host_block_tables.copy(), batch.host_context_lens.copy()))

    gc.collect()
    gc.disable()
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        run(args.warmup + j)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for j in range(args.steps):  # the event pass: kernel durations and byte counts
        run(args.warmup + args.steps + j, j)
    torch.cuda.synchronize()
    gc.enable()
    dec_s = sum(a.elapsed_time(b) for a, b in ev_dec) / args.steps / 1e3
    copy_s = sum(a.elapsed_time(b) for a, b in ev_copy) / args.steps / 1e3
    dec_bytes = sum(int(lens.sum()) for _, lens in log_tables) / args.steps * row_bytes * 2
    # HBM bytes: beams of one request share all but their last blocks, so each distinct block once
    uniq_bytes = sum(unique_rows(tab, lens) for tab, lens in log_tables) / args.steps * row_bytes * 2
    # copy traffic: the rows in use of each copied block, read and written, for K and V
    copy_bytes = sum(log_rows) / args.steps * row_bytes * 2 * 2
    dec_gbs, copy_gbs = dec_bytes / dec_s / 1e9, copy_bytes / max(copy_s, 1e-12) / 1e9
    uniq_gbs = uniq_bytes / dec_s / 1e9
    log(f"[bench] beam: {NR} requests x {NBM} beams; {sum(log_copies) / args.steps:.1f} block copies/step "
        f"({copy_bytes / 1e6:.1f} MB, {copy_s * 1e6:.1f} us, {copy_gbs:.0f} GB/s); decode {dec_s * 1e6:.1f} us "
        f"({uniq_gbs:.0f} GB/s of distinct blocks, {dec_gbs:.0f} GB/s counting every beam's reads); "
        f"step {elapsed / args.steps * 1e3:.3f} ms")
    return dict(
        metric="beam-search decode: tokens/s (one per beam) + decode KV GB/s; copy-on-write GB/s",
        value=B * args.steps / elapsed, unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=elapsed / args.steps * 1e3, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16", data="synthetic",
        config=dict(workload=cfg["name"], requests=NR, beams=NBM, context=f"U[{cfg['ctx'][0]}, {cfg['ctx'][1]}]",
                    q_heads=Hq, kv_heads=Hkv, head_dim=D, block_size=256, group_splits=batch.group_splits,
                    seed=args.seed),
        attention=f"grouped by request in {sum(log_grouped)} of {len(log_grouped)} timed steps, per beam otherwise",
        decode_kernel_us=dec_s * 1e6, decode_gbs_all_beam_reads=dec_gbs,
        copies_per_step=sum(log_copies) / args.steps, copy_kernel_us=copy_s * 1e6,
        copy=dict(bound="hbm", achieved=copy_gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=copy_gbs / HBM_PEAK_GBS,
                  bytes_per_step=copy_bytes),
        roofline=dict(bound="hbm", achieved=uniq_gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=uniq_gbs / HBM_PEAK_GBS,
                      traffic=stored_traffic("decode_group_kernel" if all(log_grouped) else "decode_split_kernel",
                                             cfg["name"]),
                      kernel=("grouped decode over each request's beams" if all(log_grouped) else
                              "decode over every beam's context") + " (bytes: distinct blocks once)",
                      bytes_per_launch=uniq_bytes),
        cpu_baseline=cpu,
    )


def cpu_baseline_beam(wl, seed, cpu_seconds=20.0):
    """The oracle's beam step on slices of the requests: admit and store the prompts, fork each into
    its beams, append one token per beam with copy-on-write (block copies included), store the new
    rows, attend over every beam."""
    import workloads as W
    from oracle import allocator as OA
    from oracle import attention as OT
    cfg = wl["cfg"]
    NBM, Hkv, D = cfg["beams"], cfg["Hkv"], cfg["D"]

    def run(lo, hi):
        seqs = wl["seqs"][lo:hi]
        n = hi - lo
        nb = W.pool_blocks(cfg, wl["lens"][lo:hi]) + 2 * n * NBM
        a = OA.Allocator(nb, W.free_order(cfg, seed, nb))
        kc = np.zeros((nb, Hkv, 256, D))
        vc = np.zeros_like(kc)
        for r, s in enumerate(seqs):
            a.add_seq(r, s["tokens"])
        _, _, slots = a.prefill_slots(list(range(n)))
        kc, vc = OT.kv_store(kc, vc, np.concatenate([W.bf16_bits_to_f32(s["k"]) for s in seqs]),
                             np.concatenate([W.bf16_bits_to_f32(s["v"]) for s in seqs]), slots)
        beams = []  # step 0: every beam continues its request's prompt
        for r in range(n):
            for j in range(NBM):
                a.fork(r, n + r * NBM + j)
                beams.append(n + r * NBM + j)
            a.free_seq(r)
        inp = W.decode_step_inputs(cfg, seed, 0, n * NBM)
        res = [a.append_cow(b, int(t)) for b, t in zip(beams, inp["tokens"])]
        cop = [x for x in res if x[1] >= 0]
        kc, vc = OT.copy_blocks([kc, vc], [x[1] for x in cop], [x[2] for x in cop], [x[0] % 256 for x in cop])
        kc, vc = OT.kv_store(kc, vc, W.bf16_bits_to_f32(inp["k"]), W.bf16_bits_to_f32(inp["v"]), [x[0] for x in res])
        lens = [a.seq_len(b) for b in beams]
        OT.decode(W.bf16_bits_to_f32(inp["q"]), kc, vc, a.block_tables(beams, -(-max(lens) // 256)), lens,
                  1.0 / math.sqrt(D))
        return n * NBM

    units, wall, w, cpu_s, n = parallel_oracle(run, len(wl["lens"]), cpu_seconds)
    return dict(value=units / wall, unit="tokens/s", cores=w, kind="oracle",
                sample=f"first {n} of {len(wl['lens'])} requests x {NBM} beams: oracle block manager (forks, "
                       f"copy-on-write), block copies, store, fp64 attention; {_pool_note(w, cpu_s, wall)}")


def cpu_baseline_prefill_rows(wl, cpu_seconds=20.0):
    """Prompts longer than a chunk: the oracle's causal attention (plain definition, fp64) for the
    last rows of the longest prompt, all heads, in slices of rows."""
    from oracle import attention as OT
    import workloads as W
    cfg = wl["cfg"]
    G = cfg["Hq"] // cfg["Hkv"]
    p = max(wl["prompts"], key=lambda x: len(x["tokens"]))
    L = len(p["tokens"])
    k, v, q = (W.bf16_bits_to_f32(p[x]).astype(np.float64) for x in ("k", "v", "q"))
    scale = 1.0 / math.sqrt(cfg["D"])

    def run(lo, hi):
        for n in range(lo, hi):
            pos = L - 1 - n
            for h in range(cfg["Hq"]):
                OT.attend(q[pos, h], k[:pos + 1, h // G], v[:pos + 1, h // G], scale)
        return hi - lo

    units, wall, w, cpu_s, n = parallel_oracle(run, L, cpu_seconds)
    return dict(value=units / wall, unit="prefill tokens/s", cores=w, kind="oracle",
                sample=f"last {n} rows of the {L}-token prompt, all {cfg['Hq']} heads: fp64 causal attention; "
                       f"{_pool_note(w, cpu_s, wall)}")


def cpu_baseline_prefill(wl, cpu_seconds=20.0):
    """The oracle's chunked prefill (its block manager, store, fp64 attention) on slices of the
    prompts; a slice's prompts share prefix blocks with each other only, so each slice computes
    the tokens it finds uncached, and those are what is counted."""
    import workloads as W
    from oracle.steps import prefill_run
    cfg = wl["cfg"]

    def run(lo, hi):
        sub = dict(wl)
        sub["lens"] = wl["lens"][lo:hi]
        sub["prompts"] = wl["prompts"][lo:hi]
        sub["num_blocks"] = W.pool_blocks(cfg, sub["lens"])
        sub["free_order"] = W.free_order(cfg, wl["seed"], sub["num_blocks"])
        _, ncached, _ = prefill_run(sub)
        return sum(L - c for L, c in zip(sub["lens"], ncached))

    units, wall, w, cpu_s, n = parallel_oracle(run, len(wl["lens"]), cpu_seconds)
    return dict(value=units / wall, unit="prefill tokens/s", cores=w, kind="oracle",
                sample=f"first {n} of {len(wl['lens'])} prompts in {w} slices ({units} new tokens): oracle block "
                       f"manager + store + fp64 causal attention; {_pool_note(w, cpu_s, wall)}")


# ------------------------------------------------------------------------------------ main
# The path's five workloads; the first is the headline (top level of the default line).
ALL_WORKLOADS = ["long_decode", "tiny_fp32", "qwen3_decode", "prefill_prefix", "int8_decode"]
SUMMARY_KEYS = ("value", "unit", "ms_per_step", "dtype", "config", "roofline", "cpu_baseline", "decode_kernel_us",
                "decode_tokens_per_s_kernel", "kv_gbs", "prefill_kernel_us", "prefill_tflops", "host_admit_us")


def bench_all(args):
    """Every workload of the path: inputs generated and the oracle baselines timed first (before the
    GPU is touched), then each workload on the GPU.  Returns one line: the headline workload at the
    top level, every workload under ``configs``."""
    import workloads as W
    cfgs = {n: W.config(n) for n in ALL_WORKLOADS}
    wls, cpus = {}, {}
    for n, cfg in cfgs.items():
        t0 = time.time()
        wls[n] = (W.prefill_workload if cfg["kind"] == "prefill" else W.decode_workload)(cfg, args.seed)
        log(f"[bench] generated {n} in {time.time() - t0:.1f}s")
        if not args.no_cpu_baseline:
            cpus[n] = (cpu_baseline_prefill(wls[n], args.cpu_seconds) if cfg["kind"] == "prefill" else
                       cpu_baseline_decode(wls[n], 0, args.cpu_seconds))
            log(f"[bench] oracle baseline {n}: {cpus[n]['value']:.4g} {cpus[n]['unit']} ({cpus[n]['sample']})")
    res = {}
    for n in [x for x in ("tiny_fp32", "qwen3_decode", "prefill_prefix", "long_decode", "int8_decode")]:
        fn = bench_prefill if cfgs[n]["kind"] == "prefill" else bench_decode
        res[n] = fn(args, cfgs[n], wls[n], cpus.get(n))
        wls[n] = None  # free the host copy
        r = res[n]["roofline"]
        log(f"[bench] {n}: {res[n]['value']:.4g} {res[n]['unit']}, {r['achieved']:.1f} {r['unit']} "
            f"({100 * r['frac']:.1f}% of peak)")
    top = dict(res[ALL_WORKLOADS[0]])
    top["configs"] = {n: {k: res[n][k] for k in SUMMARY_KEYS if k in res[n]}
                      for n in ("tiny_fp32", "qwen3_decode", "prefill_prefix", "long_decode", "int8_decode")}
    return top


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.prof_dir, args.prof_cmd, args.prof_workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch
    import workloads as W
    # device_count() does not initialise the GPU: the oracle baselines fork worker processes first
    if torch.cuda.device_count() < 1:
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calib:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_read": n, "copy_calib_bytes_written": n, "launches": 5}), flush=True)
        return
    if args.config is None:
        res = bench_all(args)
    else:
        cfg = W.config(args.config)
        if cfg["kind"] == "decode":
            res = bench_decode(args, cfg)
        elif cfg["kind"] == "store":
            res = bench_int8_store(args, cfg)
        elif cfg["kind"] == "beam":
            if args.requests > 0:
                cfg = W.config(args.config, B=args.requests)
            res = bench_beam(args, cfg)
        else:
            res = bench_prefill(args, cfg)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
