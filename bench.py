"""Benchmark of one collective-reuse round on one MI355X.

A step is one pass of the whole hot path over one synthetic round held in
HBM: batched RoPE re-rotation of the shared K for all agents and layers,
the check-layer deviation pass with important-position selection and Master
choice, the Master-Mirror diff encode, and the fused restore + decode
attention of every agent and layer.  The dense restore-then-attend
comparator is timed on the same round outside the step.

Prints ONE JSON line (see the fields below).  Default workload: the
Qwen2.5-14B-shaped full round (10 agents, 48 layers, 8 KV heads x 128,
40 query heads, bf16, 4K-8K-token contexts).
"""

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prewarm", type=float, default=1.5,
                    help="seconds of untimed steps run before each configuration's warm-up steps, so that the "
                         "GPU's clocks have settled when the timed steps start")
    ap.add_argument("--config", default="qwen14b_round")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only --config (not the 7B round, 14B round and 64-agent round beside it)")
    ap.add_argument("--no-per-config-cpu", action="store_true",
                    help="skip the oracle timings of the per-config workloads other than --config")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not read the 1 GiB scratch between timed steps")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-transfer", action="store_true",
                    help="skip the transfer-path restore measurement (Master and diffs in pinned host memory)")
    ap.add_argument("--no-serial", action="store_true",
                    help="skip the serial per-agent comparator (one-agent re-rotation and selection per agent)")
    ap.add_argument("--sq-summary", nargs=2, metavar=("SQ_CSV", "KERNEL_STATS_CSV"),
                    help="summarise a rocprofv3 --pmc run of SQ counters (MFMA/VALU/LDS use per kernel) "
                         "with a kernel-trace run's durations; runs no GPU work")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the paged-layout measurement (the four calls over 16-token pages)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling rocprofv3 byte counters)")
    ap.add_argument("--pmc-summary", nargs="+", metavar="CSV",
                    help="summarise two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, "
                         "both with --calib-copy) into HBM bytes per entry point and record them in "
                         "profiles/traffic.json; runs no GPU work")
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_STATS_CSV", "BENCH_LOG"),
                    help="summarise a rocprofv3 --kernel-trace --stats run of this script: per-kernel "
                         "average durations and each entry point's sum next to the HIP-event stage times "
                         "of the run's JSON line; runs no GPU work")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "collective_kv_cache_amd", "csrc")


# hipEventDisableSystemFence: the event skips the system-scope fence (an L2
# writeback and invalidate) when it is recorded.  The HIP runtime documents
# the flag for events used only for timing; with default events each
# stage boundary also pays for that fence (~1.5-2.5 us per stage here).
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvent:
    """A timing event on the HIP runtime that torch loaded, created with
    hipEventDisableSystemFence, recorded on torch's current stream (the stream
    the library's kernels are launched on).  Same use as torch.cuda.Event:
    record(), then elapsed_time(later_event) in ms after a synchronize."""
    _lib = None

    def __init__(self):
        import ctypes
        import torch

        if HipEvent._lib is None:
            # the HIP runtime this process has loaded (torch's, which the
            # library's kernels also run on); dlopen of its path returns it
            path = None
            try:
                with open("/proc/self/maps") as f:
                    for ln in f:
                        if "libamdhip64.so" in ln:
                            path = ln.split()[-1]
                            break
            except OSError:
                pass
            lib = ctypes.CDLL(path or os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvent._lib = lib
        self._ct = ctypes
        self._h = ctypes.c_void_p()
        rc = HipEvent._lib.hipEventCreateWithFlags(ctypes.byref(self._h), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        import torch

        rc = HipEvent._lib.hipEventRecord(self._h, self._ct.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end: "HipEvent") -> float:
        ms = self._ct.c_float()
        rc = HipEvent._lib.hipEventElapsedTime(self._ct.byref(ms), self._h, end._h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        # at interpreter exit the runtime may already be torn down: leave the
        # event to the process's end then
        if HipEvent._lib is not None and self._h and not sys.is_finalizing():
            HipEvent._lib.hipEventDestroy(self._h)
# C-ABI entry point of each stage (one call per step; its kernels run back to back)
ENTRY = {"rerotate": "tdx_rerotate", "select": "tdx_select_important", "encode": "tdx_diff_encode",
         "restore_attn": "tdx_restore_attn"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_hash() -> str:
    """sha256 over the HIP sources, to tell whether recorded counters still
    describe the kernels being run."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(entry: str, workload: str):
    """HBM bytes per call of `entry` from the rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs recorded in profiles/traffic.json, or None when absent or taken on
    other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(entry)
    if not r or r.get("workload") != workload or r.get("src_sha256") != source_hash():
        return None
    return int(r["fetch_bytes"]) + int(r["write_bytes"])


# kernels of each timed entry point (one call of the entry point launches each
# of them once); the dense comparator's kernels run outside the step
ENTRY_KERNELS = {
    "tdx_rerotate": ("rerotate_kernel",),
    "tdx_select_important": ("deviation_kernel", "select_kernel"),
    "tdx_diff_encode": ("flag_kernel", "rows_kernel", "offsets_kernel", "index_kernel", "index_rows_kernel",
                        "copy_kernel"),
    "tdx_restore_attn": ("shared_kernel",
                         "stream_plan_kernel<0>", "stream_kernel<unsigned short, 128, 0",
                         "stream_kernel<unsigned short, 64, 0", "merge_kernel<unsigned short, 128, 0>",
                         "merge_kernel<unsigned short, 64, 0>"),
}


def _short_kernel(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0].replace("tdx::", "")


def _entry_of(kernel: str):
    if kernel.rstrip().endswith("true>"):
        return None  # a paged-layout variant: not part of the timed step
    for entry, pats in ENTRY_KERNELS.items():
        if any(kernel.startswith(p) for p in pats):
            return entry
    return None


def pmc_summary(fetch_csv: str, write_csv: str, workload: str, bench_log: str = None):
    """HBM bytes per dispatch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB),
    scaled by what the same counters read for the 1 GiB calibration copy."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        vals, by_id = defaultdict(list), {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                k = _short_kernel(r["Kernel_Name"])
                vals[k].append(float(r["Counter_Value"]) * 1024.0)
                by_id[r["Dispatch_Id"]] = (k, float(r["Counter_Value"]) * 1024.0)
        return vals, by_id

    (fetch, fetch_id), (write, write_id) = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    gib = float(1 << 30)
    # the calibration copies: copy dispatches that wrote ~1 GiB; the two runs
    # launch the same dispatches in the same order, so the fetch run's
    # dispatches of the same ids are the same copies
    calib = [i for i, (k, v) in write_id.items() if "copy" in k.lower() and abs(v - gib) < 0.05 * gib]
    calib = [i for i in calib if i in fetch_id and "copy" in fetch_id[i][0].lower()]
    if not calib:
        raise SystemExit("no 1 GiB calibration copy found: run the --pmc passes with --calib-copy")
    ck = write_id[calib[0]][0]
    f_scale = gib / (sum(fetch_id[i][1] for i in calib) / len(calib))
    w_scale = gib / (sum(write_id[i][1] for i in calib) / len(calib))
    print(f"calibration ({ck}): FETCH_SIZE x {f_scale:.3f}, WRITE_SIZE x {w_scale:.3f}")
    print(f"{'kernel (per dispatch, mean)':62s} {'read_MB':>10s} {'written_MB':>11s}")
    rec = {}
    for k in sorted(set(fetch) | set(write)):
        e = _entry_of(k)
        if e is None:
            continue
        fb = f_scale * sum(fetch.get(k, [0])) / max(1, len(fetch.get(k, [0])))
        wb = w_scale * sum(write.get(k, [0])) / max(1, len(write.get(k, [0])))
        print(f"{k[:62]:62s} {fb / 1e6:10.1f} {wb / 1e6:11.1f}")
        r = rec.setdefault(e, {"workload": workload, "fetch_bytes": 0, "write_bytes": 0,
                               "src_sha256": source_hash(), "fetch_scale": round(f_scale, 4),
                               "write_scale": round(w_scale, 4)})
        r["fetch_bytes"] += int(fb)
        r["write_bytes"] += int(wb)
    for e, r in rec.items():
        print(f"{e:24s} read {r['fetch_bytes'] / 1e9:7.3f} GB  written {r['write_bytes'] / 1e9:7.3f} GB")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print("recorded in", os.path.relpath(TRAFFIC_FILE, ROOT))
    if bench_log:
        line = None
        for ln in open(bench_log):
            if ln.startswith("{"):
                line = json.loads(ln)
        if line:
            stage_of = {v: k for k, v in ENTRY.items()}
            print("\nentry point (per call): counted HBM bytes vs the algorithmic bytes bench.py uses:")
            for e, r in rec.items():
                cnt = (r["fetch_bytes"] + r["write_bytes"]) / 1e9
                alg = line["stages"][stage_of[e]]["alg_GB"]
                print(f"  {e:24s} counted {cnt:7.3f} GB   algorithmic {alg:7.3f} GB   ratio {cnt / alg:.3f}")


def sq_summary(sq_csv: str, stats_csv: str):
    """MFMA / VALU / LDS use per kernel from a rocprofv3 --pmc run of SQ
    counters, with each kernel's average duration from a kernel-trace run:
    MFMA% = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x kernel cycles at 2.4 GHz),
    MFMA GFLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512."""
    import csv
    from collections import defaultdict

    acc, disp = defaultdict(lambda: defaultdict(float)), defaultdict(set)
    for r in csv.DictReader(open(sq_csv)):
        k = _short_kernel(r["Kernel_Name"])
        acc[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
    us = {_short_kernel(r["Name"]): float(r["AverageNs"]) / 1e3 for r in csv.DictReader(open(stats_csv))}
    print(f"{'kernel':46s} {'us':>8s} {'MFMA%':>7s} {'MFMA_GF':>8s} {'TFLOP/s':>8s} {'VALU_inst':>10s} "
          f"{'MFMA_inst':>10s} {'LDS_inst':>9s}")
    for k in sorted(acc, key=lambda k: -us.get(k, 0.0)):
        if _entry_of(k) is None or k not in us:
            continue
        n = len(disp[k])
        c = {name: v / n for name, v in acc[k].items()}
        t = us[k]
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024 * t * 2400.0)
        gf = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 / 1e9
        print(f"{k[:46]:46s} {t:8.1f} {100 * busy:6.1f}% {gf:8.1f} {gf / t * 1e3:8.1f} "
              f"{c.get('SQ_INSTS_VALU', 0.0):10.3g} {c.get('SQ_INSTS_MFMA', 0.0):10.3g} "
              f"{c.get('SQ_INSTS_LDS', 0.0):9.3g}")
    # any other counters of the run, per dispatch, for the same kernels
    shown = {"SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
             "SQ_INSTS_LDS"}
    extra = sorted({n for k in acc for n in acc[k]} - shown)
    if extra:
        print("\nother counters, per dispatch:")
        print(f"{'kernel':46s} " + " ".join(f"{n[3:][:22]:>22s}" for n in extra))
        for k in sorted(acc, key=lambda k: -us.get(k, 0.0)):
            if _entry_of(k) is None or k not in us:
                continue
            n = len(disp[k])
            print(f"{k[:46]:46s} " + " ".join(f"{acc[k].get(x, 0.0) / n:22.4g}" for x in extra))


def trace_summary(stats_csv: str, bench_log: str):
    """Per-kernel average durations of a rocprofv3 --kernel-trace --stats run
    and each entry point's sum next to the run's HIP-event stage times."""
    import csv

    rows = list(csv.DictReader(open(stats_csv)))
    print(f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'total_us':>11s}")
    avg = {}
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        k = _short_kernel(r["Name"])
        avg[k] = float(r["AverageNs"]) / 1e3
        print(f"{k[:60]:60s} {int(r['Calls']):6d} {avg[k]:10.1f} {float(r['TotalDurationNs']) / 1e3:11.1f}")
    line = None
    for ln in open(bench_log):
        if ln.startswith("{"):
            line = json.loads(ln)
    stage_of = {v: k for k, v in ENTRY.items()}
    print("\nentry point = sum of its kernels' averages (rocprofv3) vs the HIP-event time of the stage:")
    for e in ENTRY_KERNELS:
        us = sum(v for k, v in avg.items() if _entry_of(k) == e)
        ev = line["stages"][stage_of[e]]["ms"] * 1e3 if line else float("nan")
        print(f"  {e:26s} {us:9.1f} us   bench {ev:9.1f} us")


def stage_bytes(cfg, lay, nnz_total, k):
    """Algorithmic HBM bytes of each stage (what the method must move)."""
    N, L, T, H, D, Hq = cfg.n_agents, cfg.n_layers, lay.n_tokens, cfg.n_kv_heads, cfg.head_dim, cfg.n_q_heads
    eb = cfg.elem_bytes
    kt = H * D * eb
    kv = 2 * kt
    ptot = int(lay.priv_len.sum())
    blk = 16 * kv
    diff_bytes = nnz_total * (blk + 4)
    return {
        "rerotate": L * T * kt + N * L * T * kt,
        "select": 2 * N * T * kt + 4 * N * T + 4 * T + 4 * k + 4 * N,
        # read every agent's cache once, write diff values + indices (the Master
        # stays in place)
        "encode": N * L * T * kv + diff_bytes + 4 * (N * L + 1),
        # Master once, private histories, diff records, q and out
        "restore_attn": L * T * kv + L * ptot * kv + diff_bytes + 2 * N * L * Hq * D * eb,
        # dense restore (read Master + diffs, write N dense caches) + attention over them
        "dense": (L * T * kv + diff_bytes + N * L * T * kv) + (L * ptot * kv + N * L * T * kv)
                 + 2 * N * L * Hq * D * eb,
    }


def compression(counts, master, T, H, D, eb, priv_len, L):
    """Storage of the shared region: dense N copies vs Master + diff rows."""
    import numpy as np

    counts = np.asarray(counts, dtype=np.int64)
    N = counts.shape[0]
    dense_one = L * T * H * D * 2 * eb
    row = counts * (16 * H * D * 2 * eb + 4) + 4
    mirror = row.sum(axis=1)
    per = [dense_one / float(mirror[i]) for i in range(N) if i != master]
    stored = dense_one + sum(int(mirror[i]) for i in range(N) if i != master)
    priv = int(np.sum(priv_len)) * L * H * D * 2 * eb
    return {
        "per_mirror_ratio_mean": float(np.mean(per)) if per else None,
        "group_ratio": N * dense_one / float(stored),
        "dense_shared_GB": N * dense_one / 1e9,
        "master_plus_diff_GB": stored / 1e9,
        "footprint_with_private_ratio": (N * dense_one + priv) / float(stored + priv),
        "dense_total_GB": (N * dense_one + priv) / 1e9,
        "stored_total_GB": (stored + priv) / 1e9,
    }


# ---- the oracle on the host (cpu_baseline) ----------------------------------
# The oracle runs in a pool of worker processes created before this process
# makes its first GPU call (spawned interpreters, one torch / BLAS thread
# each).  A round's layers are independent, so each worker takes whole layers:
# it draws the layer's inputs on the host (same shapes and structure as the
# GPU round) and times the oracle's stages on them.

POOL_MAX = 16  # the host's CPU share on a one-GPU machine


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def make_oracle_pool():
    """(pool, size): spawned workers, sized to the affinity mask capped at POOL_MAX."""
    import multiprocessing as mp

    n = max(1, min(len(os.sched_getaffinity(0)), POOL_MAX))
    return mp.get_context("spawn").Pool(n, initializer=_oracle_worker_init), n


def _oracle_worker_init():
    os.environ["OMP_NUM_THREADS"] = "1"
    import torch

    torch.set_num_threads(1)


def _oracle_select(name: str):
    """Check layer: the oracle's re-rotation of it (input preparation), then
    the timed deviation, top-k and Master."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O
    from workload import CONFIGS, cached_kv, from_numpy_bits, make_layout, recomputed_k, to_numpy_bits

    cfg = CONFIGS[name]
    lay = make_layout(cfg)
    with threadpool_limits(limits=1):
        kc, _ = cached_kv(cfg, lay, layers=[cfg.check_layer])
        kr = O.rerotate(to_numpy_bits(kc), lay.blk_start, lay.src_pos, lay.dst_pos, cfg.theta)[:, 0]
        kx = to_numpy_bits(recomputed_k(cfg, lay, from_numpy_bits(kr)))
        t0 = time.perf_counter()
        _, s, a = O.deviation(kr, kx)
        O.select_important(s.astype(np.float32), O.topk_count(cfg.pct, lay.n_tokens))
        m = O.choose_master(a.astype(np.float32))
        t1 = time.perf_counter()
    return m, t1 - t0


def _oracle_layer(name: str, layer: int, master: int):
    """One layer of the round: draw its inputs, then time the oracle's
    re-rotation, diff encode and restore-attention of that layer."""
    from threadpoolctl import threadpool_limits

    import oracle as O
    from workload import (CONFIGS, agent_caches, cached_kv, make_layout, private_kv, queries,
                          to_numpy_bits)

    cfg = CONFIGS[name]
    lay = make_layout(cfg)
    g0 = time.perf_counter()
    with threadpool_limits(limits=1):
        kc, vc = cached_kv(cfg, lay, layers=[layer])
        q = to_numpy_bits(queries(cfg)[:, layer:layer + 1])
        pk, pv = (to_numpy_bits(x) for x in private_kv(cfg, lay, layers=[layer]))
        ak, av = (to_numpy_bits(x) for x in agent_caches(cfg, lay, kc, vc, master))
        hk, hv = to_numpy_bits(kc), to_numpy_bits(vc)
        t0 = time.perf_counter()
        O.rerotate(hk, lay.blk_start, lay.src_pos, lay.dst_pos, cfg.theta)
        t1 = time.perf_counter()
        off, idx, dk, dv = O.diff_encode(ak, av, master)
        t2 = time.perf_counter()
        O.restore_attn(q, lay.priv_off, pk, pv, hk, hv, off, idx, dk, dv, lay.blk_start, lay.src_pos,
                       lay.dst_pos, cfg.theta, 1.0 / math.sqrt(cfg.head_dim))
        t3 = time.perf_counter()
    return {"pid": os.getpid(), "layer": layer, "draw": t0 - g0, "rerotate": t1 - t0, "encode": t2 - t1,
            "restore_attn": t3 - t2}


def cpu_baseline(pool, n_pool: int, name: str, layers=None):
    """The oracle's round time on the host's cores: the check-layer selection,
    then the round's layers spread over the pool.  value = N*T agent-tokens /
    (selection + the largest per-process sum of the layers' oracle stage
    times); drawing the inputs is not counted.  ``layers``: a bounded sample
    of the round's layers (the per-layer stages then scale by L / len)."""
    from collections import defaultdict

    from workload import CONFIGS, make_layout

    cfg = CONFIGS[name]
    lay = make_layout(cfg)
    L = cfg.n_layers
    layers = list(range(L)) if layers is None else list(layers)
    w0 = time.perf_counter()
    master, t_sel = pool.apply(_oracle_select, (name,))
    res = pool.starmap(_oracle_layer, [(name, l, master) for l in layers], chunksize=1)
    wall = time.perf_counter() - w0
    per_proc = defaultdict(float)
    for r in res:
        per_proc[r["pid"]] += r["rerotate"] + r["encode"] + r["restore_attn"]
    f = L / len(layers)
    stage = {k: sum(r[k] for r in res) * f for k in ("rerotate", "encode", "restore_attn")}
    if len(layers) == L:
        layers_s = max(per_proc.values())  # measured: the busiest process's oracle time
    else:
        # a sample: the whole round's oracle time spread over the pool, but no
        # less than one layer's
        layers_s = max(sum(stage.values()) / n_pool,
                       max(r["rerotate"] + r["encode"] + r["restore_attn"] for r in res))
    round_s = t_sel + layers_s
    sample = (f"every layer of the {name} round ({L} layers, {cfg.n_agents} agents, {lay.n_tokens} shared "
              f"tokens, the same shapes and structure as the GPU round, drawn on the host)"
              if len(layers) == L else
              f"layers {layers[0]}..{layers[-1]} of the {L} of the {name} round ({cfg.n_agents} agents, "
              f"{lay.n_tokens} shared tokens); the round's oracle time is their stage times x {L}/{len(layers)} "
              f"spread evenly over the {n_pool} processes")
    return {
        "value": cfg.n_agents * lay.n_tokens / round_s,
        "unit": "agent-tokens/s",
        "cores": len(per_proc) if len(layers) == L else n_pool,
        "kind": "oracle",
        "sample": (sample + (f"; layers spread over {len(per_proc)} worker processes, one thread each; round "
                             f"time = check-layer selection + the largest per-process sum of its layers' oracle "
                             f"stage times" if len(layers) == L else "") + "; drawing the inputs is not counted"),
        "cpu": cpu_model(),
        "round_s": round(round_s, 3),
        "oracle_cpu_s": round(t_sel + sum(stage.values()), 2),
        "stage_cpu_s": {"select": round(t_sel, 3), **{k: round(v, 2) for k, v in stage.items()}},
        "wall_s": round(wall, 2),
    }


def time_calls(fn, steps, warmup, flush):
    """Mean ms of fn() over ``steps`` calls, each after ``flush`` and timed by
    its own HIP events (the flush falls outside them)."""
    import torch

    for _ in range(warmup):
        flush()
        fn()
    evs = [(HipEvent(), HipEvent()) for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps


PCIE_H2D_GBS = 64.0  # PCIe 5.0 x16, one direction, nominal


def transfer_path(cfg, lay, shape, dl, ds, nnz, master_k, master_v, q, pk, pv, reps=3):
    """The transfer-path restore of the same round with the Master and the
    diff record in pinned host memory (outside the timed step):
      - every agent's KV for every layer in one call: bytes over PCIe / time;
      - one Mirror, layer by layer (the pages' per-Mirror per-layer latency);
      - decode attention of that Mirror over each restored layer, the only
        work a restore on a second stream could hide (its share of the
        restore time bounds what overlap can gain)."""
    import numpy as np
    import torch
    from collective_kv_cache_amd import tdx

    dev = "cuda"
    N, L, T, H, Hq, D = cfg.n_agents, cfg.n_layers, lay.n_tokens, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim
    kt = H * D * cfg.elem_bytes
    torch.cuda.synchronize()
    mk_h, mv_h = master_k.cpu().pin_memory(), master_v.cpu().pin_memory()
    off_h, idx_h = ds.off.cpu().pin_memory(), ds.idx[:max(nnz, 1)].cpu().pin_memory()
    dk_h, dv_h = ds.k[:max(nnz, 1)].cpu().pin_memory(), ds.v[:max(nnz, 1)].cpu().pin_memory()
    counts = np.diff(off_h.numpy().astype(np.int64)).reshape(N, L)
    ev = lambda: HipEvent()

    def timed(fn, n=reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # every agent, every layer
    ag = torch.arange(N, dtype=torch.int32, device=dev)
    k_all = torch.empty((N, L, T, H, D), dtype=cfg.torch_dtype, device=dev)
    v_all = torch.empty_like(k_all)
    ws_all = torch.empty(tdx.restore_transfer_workspace(shape, dl, N, 0, L), dtype=torch.uint8, device=dev)
    ms_all = timed(lambda: tdx.restore_transfer(shape, dl, mk_h, mv_h, off_h, idx_h, dk_h, dv_h, ag, 0, L,
                                                k_all, v_all, ws_all))
    pcie_all = L * T * 2 * kt + int(counts.sum()) * (16 * 2 * kt + 4) + 4 * (N * L + 1)
    del k_all, v_all
    # one Mirror (the one with the most diff blocks), layer by layer
    mir = int(np.argmax(counts.sum(axis=1)))
    a1 = torch.tensor([mir], dtype=torch.int32, device=dev)
    k1 = torch.empty((1, L, T, H, D), dtype=cfg.torch_dtype, device=dev)
    v1 = torch.empty_like(k1)
    ws1 = torch.empty(tdx.restore_transfer_workspace(shape, dl, 1, 0, 1), dtype=torch.uint8, device=dev)
    restore_l = lambda l: tdx.restore_transfer(shape, dl, mk_h, mv_h, off_h, idx_h, dk_h, dv_h, a1, l, l + 1,
                                               k1, v1, ws1)
    ms_layers = timed(lambda: [restore_l(l) for l in range(L)])
    pcie_mirror = L * T * 2 * kt + int(counts[mir].sum()) * (16 * 2 * kt + 4)
    # decode attention of that Mirror over each restored layer (one agent, one
    # layer per call): the work a second stream could overlap with the restore
    shape1 = tdx.Shape(1, H, Hq, D, cfg.torch_dtype, cfg.theta)
    dl1 = tdx.RoundLayout(lay.blk_start, lay.src_pos, lay.dst_pos[mir:mir + 1], dev)
    p0, p1 = int(lay.priv_off[mir]), int(lay.priv_off[mir + 1])
    po1 = torch.tensor([0, p1 - p0], dtype=torch.int32, device=dev)
    out1 = torch.empty((1, 1, Hq, D), dtype=cfg.torch_dtype, device=dev)
    ws_a = torch.empty(max(tdx.decode_attn_dense_workspace(shape1, dl1, max(p1 - p0, 1)), 16), dtype=torch.uint8,
                       device=dev)
    pk1 = [pk[l:l + 1, p0:p1] if p1 > p0 else pk[l:l + 1, :1] for l in range(L)]
    pv1 = [pv[l:l + 1, p0:p1] if p1 > p0 else pv[l:l + 1, :1] for l in range(L)]
    attn_l = lambda l: tdx.decode_attn_dense(shape1, dl1, q[mir:mir + 1, l:l + 1], po1, pk1[l], pv1[l], p1 - p0,
                                             k1[:, l:l + 1], v1[:, l:l + 1], out=out1, ws=ws_a)
    attn_ms = timed(lambda: [attn_l(l) for l in range(L)])
    return {
        "source": "pinned host memory (Master + diff record), read by the restore kernel over PCIe",
        "all_agents_ms": round(ms_all, 3),
        "all_agents_pcie_GB": round(pcie_all / 1e9, 4),
        "all_agents_GBps": round(pcie_all / (ms_all * 1e-3) / 1e9, 2),
        "frac_pcie_peak": round(pcie_all / (ms_all * 1e-3) / 1e9 / PCIE_H2D_GBS, 4),
        "dense_pcie_GB_avoided": round(N * L * T * 2 * kt / 1e9, 3),
        "mirror": mir,
        "ms_per_mirror_per_layer": round(ms_layers / L, 4),
        "mirror_GBps": round(pcie_mirror / (ms_layers * 1e-3) / 1e9, 2),
        "mirror_attend_ms_per_layer": round(attn_ms / L, 4),
        "attend_over_restore": round(attn_ms / ms_layers, 4),
    }


def _to_pool(seqs, gen):
    """Per-sequence [L][n][Hkv][D] device tensors -> (pool [L][P][16][Hkv][D],
    page table [rows][stride]) with the pages in a seeded random order."""
    import torch

    L, _, H, D = seqs[0].shape
    dev = seqs[0].device
    npg = [(s.shape[1] + 15) // 16 for s in seqs]
    n_pages = max(sum(npg), 1)
    perm = torch.randperm(n_pages, generator=gen).to(dev)
    pool = torch.zeros((L, n_pages, 16, H, D), dtype=seqs[0].dtype, device=dev)
    stride = max(max(npg), 1)
    pages = torch.zeros((len(seqs), stride), dtype=torch.int32, device=dev)
    k = 0
    for r, s in enumerate(seqs):
        n, ids = s.shape[1], perm[k:k + npg[r]]
        k += npg[r]
        pages[r, :npg[r]] = ids.to(torch.int32)
        full = n // 16
        if full:
            pool[:, ids[:full]] = s[:, :full * 16].reshape(L, full, 16, H, D)
        if n > full * 16:
            pool[:, ids[-1], :n - full * 16] = s[:, full * 16:]
    return pool, pages


def paged_path(cfg, lay, shape, shape1, dl, kc, kr, kx, k, msel, ak, av, q, po, pk, pv, max_priv, out_ref,
               steps, warmup, stage_ms, nnz, flush):
    """The four calls over 16-token pages (shuffled page order), timed like the
    step's stages, with the same algorithmic bytes (the paged record holds a
    page ID per entry instead of a value copy)."""
    import torch

    from collective_kv_cache_amd import tdx

    N, L, T, H, D, Hq = cfg.n_agents, cfg.n_layers, lay.n_tokens, cfg.n_kv_heads, cfg.head_dim, cfg.n_q_heads
    gen = torch.Generator(device="cpu").manual_seed(0)
    cpool, cpages = _to_pool([kc], gen)
    rpool, rpages = _to_pool([kr[i] for i in range(N)], gen)
    kpool, apages = _to_pool([ak[i] for i in range(N)], gen)
    vpool = torch.empty_like(kpool)
    nbp = T // 16
    for i in range(N):  # the V pool under the same table
        vpool[:, apages[i].long()] = av[i].reshape(L, nbp, 16, H, D)
    pof = lay.priv_off
    ppk, ppages = _to_pool([pk[:, pof[i]:pof[i + 1]] for i in range(N)], gen)
    ppv = torch.empty_like(ppk)
    for i in range(N):
        n = int(pof[i + 1] - pof[i])
        full = n // 16
        ids = ppages[i, :(n + 15) // 16].long()
        if full:
            ppv[:, ids[:full]] = pv[:, pof[i]:pof[i] + full * 16].reshape(L, full, 16, H, D)
        if n > full * 16:
            ppv[:, ids[-1], :n - full * 16] = pv[:, pof[i] + full * 16:pof[i + 1]]
    cached = tdx.PagedKV(cpool, None, cpages)
    rview = tdx.PagedKV(rpool, None, rpages)
    agents = tdx.PagedKV(kpool, vpool, apages)
    priv = tdx.PagedKV(ppk, ppv, ppages)
    sel = tdx.select_important_paged(shape1, dl, rview, kx, k, cfg.check_layer)
    cap = int(math.ceil(0.35 * (N - 1) * L * nbp))
    pd = tdx.diff_encode_paged(shape, dl, msel, agents, cap_blocks=cap)
    out = tdx.restore_attn_paged(shape, dl, q, po, priv, max_priv, agents, msel, pd)
    ws_s = torch.empty(max(tdx.select_workspace(shape1, dl), 16), dtype=torch.uint8, device=kc.device)
    ws_e = torch.empty(max(tdx.encode_workspace(shape, dl), 16), dtype=torch.uint8, device=kc.device)
    ws_a = torch.empty(max(tdx.restore_attn_workspace(shape, dl, max_priv), 16), dtype=torch.uint8,
                       device=kc.device)
    calls = {
        "rerotate": lambda: tdx.rerotate_paged(shape, dl, cached, rview),
        "select": lambda: tdx.select_important_paged(shape1, dl, rview, kx, k, cfg.check_layer, out=sel, ws=ws_s),
        "encode": lambda: tdx.diff_encode_paged(shape, dl, msel, agents, out=pd, check=False, ws=ws_e),
        "restore_attn": lambda: tdx.restore_attn_paged(shape, dl, q, po, priv, max_priv, agents, msel, pd, out=out,
                                                       ws=ws_a),
    }
    byts = stage_bytes(cfg, lay, nnz, k)
    kv = 2 * H * D * cfg.elem_bytes
    byts["encode"] = N * L * T * kv + nnz * 8 + 4 * (N * L + 1)  # index + page ID per entry
    res = {}
    for name, fn in calls.items():
        ms = time_calls(fn, steps, warmup, flush)
        gbs = byts[name] / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "alg_GB": round(byts[name] / 1e9, 4), "GBps": round(gbs, 1),
                     "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                     "paged_over_contiguous": round(ms / stage_ms[name], 3)}
    bits = (lambda t: t.view(torch.int16)) if out.dtype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    res["nnz_equal"] = pd.nnz() == nnz
    res["restore_bit_identical"] = bool(torch.equal(bits(out), bits(out_ref)))
    res["layout"] = "16-token pages in a seeded random order; the diff record names pages (no value copies)"
    del cpool, rpool, kpool, vpool, ppk, ppv
    torch.cuda.empty_cache()
    return res


def graph_step(step, steps, warmup, eager_ms, out, flush):
    """One step captured in a HIP graph (outputs and workspaces preallocated,
    no allocation or memset inside the calls) and replayed."""
    import torch

    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    ms = time_calls(g.replay, steps, warmup, flush)
    bits = (lambda t: t.view(torch.int16)) if out.dtype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    same = bool(torch.equal(bits(out), bits(ref)))
    del g
    return {"ms_per_step": round(ms, 4), "eager_ms_per_step": round(eager_ms, 4),
            "graph_over_eager": round(ms / eager_ms, 4), "restore_bit_identical": same}


def serial_path(shape, lay, kc, kx, k, check_layer, kr, steps, warmup, collective_ms, flush):
    """N one-agent launches of re-rotation and selection (the per-request
    path) against the collective round's one launch of each."""
    import torch

    from collective_kv_cache_amd.serial import SerialReuse

    ser = SerialReuse(shape, lay.blk_start, lay.src_pos, lay.dst_pos, k, kr.device)
    kr_s = torch.empty_like(kr)
    ms = time_calls(lambda: ser.run(kc, kx, check_layer, kr_s), steps, warmup, flush)
    same = bool(torch.equal(kr_s.view(torch.int16) if kr.dtype == torch.bfloat16 else kr_s.view(torch.int32),
                            kr.view(torch.int16) if kr.dtype == torch.bfloat16 else kr.view(torch.int32)))
    del kr_s
    return {"ms": round(ms, 4), "launches": 2 * lay.n_agents, "collective_ms": round(collective_ms, 4),
            "serial_over_collective": round(ms / collective_ms, 3),
            "rerotate_bit_identical": same,
            "note": "kernel time only; the pages' 2.57x includes model recompute"}


FLUSH_BYTES = 1 << 30  # read between timed steps: more than the last-level cache and the L2s hold


def measure(name, args, legs: bool, flush):
    """One round of workload ``name`` in HBM: ``args.prewarm`` seconds of
    untimed steps, ``args.warmup`` warm-up steps, then ``args.steps`` timed
    steps, each after a cache flush and bracketed by its own HIP events (the
    flush falls outside them).  With ``legs``, the graph replay, serial,
    paged and transfer legs follow; the dense comparator runs unless
    --no-dense."""
    import numpy as np
    import torch

    from collective_kv_cache_amd import tdx
    from workload import (CONFIGS, make_layout, cached_kv, agent_caches, queries, private_kv,
                          recomputed_k)

    dev = "cuda"
    cfg = CONFIGS[name]
    lay = make_layout(cfg)
    N, L, T, H, Hq, D = cfg.n_agents, cfg.n_layers, lay.n_tokens, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim
    shape = tdx.Shape(L, H, Hq, D, cfg.torch_dtype, cfg.theta)
    shape1 = shape.with_layers(L)
    dl = tdx.RoundLayout(lay.blk_start, lay.src_pos, lay.dst_pos, dev)
    k = tdx.topk_count(cfg.pct, T)
    max_priv = int(lay.priv_len.max())

    # ---- inputs, drawn directly in HBM
    kc, vc = cached_kv(cfg, lay, device=dev)
    q = queries(cfg, device=dev)
    pk, pv = private_kv(cfg, lay, device=dev)
    po = torch.as_tensor(lay.priv_off, device=dev)
    kr = torch.empty((N, L, T, H, D), dtype=cfg.torch_dtype, device=dev)
    tdx.rerotate(shape, dl, kc, out=kr)
    kx = recomputed_k(cfg, lay, kr[:, cfg.check_layer].contiguous())
    sel = tdx.select_important(shape1, dl, kr, kx, k, check_layer=cfg.check_layer)
    master = int(sel["master"].item())
    ak, av = agent_caches(cfg, lay, kc, vc, master)
    nb = T // 16
    cap = int(math.ceil(0.35 * (N - 1) * L * nb))  # the Mirrors differ in at most 20% of blocks
    # the Master keeps its own cache: no dense copy, restore reads it in place
    ds = tdx.diff_encode(shape, dl, sel["master"], ak, av, cap_blocks=cap, check=True, master_copy=False)
    out = tdx.restore_attn(shape, dl, q, po, pk, pv, max_priv, ak, av, ds, master_sel=sel["master"])
    ws_sel = torch.empty(max(tdx.select_workspace(shape1, dl), 16), dtype=torch.uint8, device=dev)
    ws_enc = torch.empty(max(tdx.encode_workspace(shape, dl), 16), dtype=torch.uint8, device=dev)
    ws_att = torch.empty(max(tdx.restore_attn_workspace(shape, dl, max_priv), 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    nnz = ds.nnz()
    counts = np.diff(ds.off.cpu().numpy().astype(np.int64)).reshape(N, L)

    stages = ["rerotate", "select", "encode", "restore_attn"]

    def step(ev=None):
        def mark(j):
            if ev is not None:
                ev[j].record()
        mark(0)
        tdx.rerotate(shape, dl, kc, out=kr)
        mark(1)
        tdx.select_important(shape1, dl, kr, kx, k, check_layer=cfg.check_layer, out=sel, ws=ws_sel)
        mark(2)
        tdx.diff_encode(shape, dl, sel["master"], ak, av, out=ds, check=False, ws=ws_enc)
        mark(3)
        tdx.restore_attn(shape, dl, q, po, pk, pv, max_priv, ak, av, ds, out=out, ws=ws_att,
                         master_sel=sel["master"])
        mark(4)

    def timed_steps(fn, steps, nev):
        """fn(events) per step; a flush before each step, outside its events."""
        evs = [[HipEvent() for _ in range(nev)] for _ in range(steps)]
        torch.cuda.synchronize()
        for s_ in range(steps):
            flush()
            fn(evs[s_])
        torch.cuda.synchronize()
        return evs

    # untimed steps until the GPU has run this round's work for args.prewarm
    # seconds (its clocks settle under sustained load; measured: 7B and
    # 64-agent steps ~2 % faster after 1.5 s than straight after set-up)
    t_pre = time.time()
    while time.time() - t_pre < args.prewarm:
        flush()
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        flush()
        step()
    evs = timed_steps(step, args.steps, 5)
    per_step = [evs[s_][0].elapsed_time(evs[s_][4]) for s_ in range(args.steps)]
    ms_step = float(np.mean(per_step))
    stage_all = {nm: [evs[s_][j].elapsed_time(evs[s_][j + 1]) for s_ in range(args.steps)]
                 for j, nm in enumerate(stages)}
    stage_ms = {nm: float(np.mean(v)) for nm, v in stage_all.items()}
    if ds.nnz() != nnz or nnz > cap:
        raise RuntimeError("diff encode changed between steps or overflowed")

    # ---- dense comparator on the same round (outside the step)
    byts = stage_bytes(cfg, lay, nnz, k)
    dense = None
    if not args.no_dense:
        kd = torch.empty((N, L, T, H, D), dtype=cfg.torch_dtype, device=dev)
        vd = torch.empty_like(kd)
        outd = torch.empty_like(out)
        ws_d = torch.empty(max(tdx.decode_attn_dense_workspace(shape, dl, max_priv), 16), dtype=torch.uint8,
                           device=dev)

        def dense_step(ev):
            ev[0].record()
            tdx.restore_dense(shape, dl, ak, av, ds, kd, vd, master_sel=sel["master"])
            ev[1].record()
            tdx.decode_attn_dense(shape, dl, q, po, pk, pv, max_priv, kd, vd, out=outd, ws=ws_d)
            ev[2].record()

        for _ in range(max(1, args.warmup)):
            flush()
            dense_step([HipEvent() for _ in range(3)])
        devs = timed_steps(dense_step, args.steps, 3)
        dense_ms = float(np.mean([e[0].elapsed_time(e[2]) for e in devs]))
        restore_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in devs]))
        diff = (outd.float() - out.float()).abs().max().item()
        gbs = byts["dense"] / (dense_ms * 1e-3) / 1e9
        dense = {"ms": round(dense_ms, 4), "restore_ms": round(restore_ms, 4),
                 "attend_ms": round(dense_ms - restore_ms, 4), "fused_ms": round(stage_ms["restore_attn"], 4),
                 "speedup_fused_vs_dense": round(dense_ms / stage_ms["restore_attn"], 3),
                 "alg_bytes_dense_over_fused": round(byts["dense"] / byts["restore_attn"], 3),
                 "max_abs_fused_minus_dense": diff, "alg_GB": round(byts["dense"] / 1e9, 3),
                 "GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del kd, vd, outd

    graph = serial = paged = transfer = None
    if legs and not args.no_graph:
        graph = graph_step(step, args.steps, max(1, args.warmup), ms_step, out, flush)
    if legs and not args.no_serial:
        serial = serial_path(shape1, lay, kc, kx, k, cfg.check_layer, kr, args.steps,
                             max(1, args.warmup), stage_ms["rerotate"] + stage_ms["select"], flush)
    if legs and not args.no_paged:
        paged = paged_path(cfg, lay, shape, shape1, dl, kc, kr, kx, k, sel["master"], ak, av, q, po, pk, pv,
                           max_priv, out, args.steps, max(1, args.warmup), stage_ms, nnz, flush)
    if legs and not args.no_transfer:
        transfer = transfer_path(cfg, lay, shape, dl, ds, nnz, ak[master], av[master], q, pk, pv)

    stage_rep = {}
    for nm in stages:
        gbs = byts[nm] / (stage_ms[nm] * 1e-3) / 1e9
        stage_rep[nm] = {"ms": round(stage_ms[nm], 4), "ms_median": round(float(np.median(stage_all[nm])), 4),
                         "ms_min": round(float(np.min(stage_all[nm])), 4), "alg_GB": round(byts[nm] / 1e9, 4),
                         "GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    res = {
        "cfg": cfg, "lay": lay, "k": k, "nnz": nnz, "master": master, "ms_step": ms_step,
        "stage_ms": stage_ms, "stages": stage_rep, "bytes": byts, "dense": dense, "graph": graph,
        "serial": serial, "paged": paged, "transfer": transfer,
        "compression": compression(counts, master, T, H, D, cfg.elem_bytes, lay.priv_len, L),
    }
    del kc, vc, q, pk, pv, kr, kx, ak, av, ds, out, ws_sel, ws_enc, ws_att
    torch.cuda.empty_cache()
    return res


def config_summary(r):
    """The per-workload entry of the JSON line."""
    cfg, lay = r["cfg"], r["lay"]
    N, T = cfg.n_agents, lay.n_tokens
    return {
        "n_agents": N, "n_layers": cfg.n_layers, "n_kv_heads": cfg.n_kv_heads, "shared_tokens": T,
        "private_tokens_total": int(lay.priv_len.sum()), "diff_blocks": r["nnz"],
        "ms_per_step": round(r["ms_step"], 4),
        "agent_tokens_per_s": N * T / (r["ms_step"] * 1e-3),
        "stages": {k: {f: v[f] for f in ("ms", "ms_median", "GBps", "frac_hbm_peak")} for k, v in r["stages"].items()},
        "dense_comparator": None if r["dense"] is None else {
            f: r["dense"][f] for f in ("ms", "speedup_fused_vs_dense", "alg_bytes_dense_over_fused", "frac_hbm_peak")},
    }


PER_CONFIG = ("qwen7b_round", "qwen14b_round", "qwen7b_scaleout")
# bounded oracle samples for the per-workload CPU figures (the 64-agent round's
# full oracle pass takes several CPU-minutes)
CPU_SAMPLE_LAYERS = {"qwen7b_scaleout": range(0, 4)}


def main():
    args = parse()
    if args.pmc_summary:
        if len(args.pmc_summary) not in (2, 3):
            raise SystemExit("--pmc-summary FETCH_CSV WRITE_CSV [BENCH_LOG]")
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.config, *args.pmc_summary[2:])
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.sq_summary:
        sq_summary(*args.sq_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the collective reuse path here runs on a single "
              "MI355X (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    # the oracle's worker processes start before this process touches the GPU
    pool = n_pool = None
    if not args.no_cpu_baseline:
        pool, n_pool = make_oracle_pool()

    import torch

    dev = "cuda"
    flush_buf = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device=dev)

    def read_flush():
        # Reading 1 GiB evicts the previous step's lines from the 256 MB
        # last-level cache and the L2s, and the dirty ones are written back
        # here, outside the timed region.  A scratch write would instead
        # leave the caches full of dirty lines whose write-back the next
        # step's first kernel pays for.
        flush_buf.sum()

    flush = read_flush if not args.no_flush else (lambda: None)

    if args.calib_copy:
        # a plain copy of known size (1 GiB read + 1 GiB written) for scaling
        # the FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 --pmc run
        csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)
        for _ in range(3):
            cdst.copy_(csrc)
        torch.cuda.synchronize()
        del csrc, cdst

    main_r = measure(args.config, args, legs=True, flush=flush)
    per_config = {args.config: config_summary(main_r)}
    for nm in ([] if args.no_per_config else [c for c in PER_CONFIG if c != args.config]):
        per_config[nm] = config_summary(measure(nm, args, legs=False, flush=flush))

    cfg, lay = main_r["cfg"], main_r["lay"]
    N, L, T, H, Hq, D = cfg.n_agents, cfg.n_layers, lay.n_tokens, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim
    stage_ms, stage_rep, byts = main_r["stage_ms"], main_r["stages"], main_r["bytes"]
    stages = list(stage_rep)
    dom = max(stages, key=lambda n: stage_ms[n])
    reuse_ms = stage_ms["rerotate"] + stage_ms["select"]
    agent_tokens = N * T
    ms_step = main_r["ms_step"]
    res = {
        "metric": "collective reuse agent-tokens/s; fused restore-attn GB/s (% of HBM peak)",
        "value": agent_tokens / (ms_step * 1e-3),
        "unit": "agent-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) K/V/q, generated in HBM)",
        "config": {"workload": cfg.name, "n_agents": N, "n_layers": L, "n_kv_heads": H,
                   "n_q_heads": Hq, "head_dim": D, "shared_tokens": T,
                   "private_tokens_total": int(lay.priv_len.sum()), "select_k": main_r["k"],
                   "diff_blocks": main_r["nnz"], "master": main_r["master"], "parallelism": "single GPU"},
        "timing": (f"each step timed by its own HIP events on the launch stream (created with "
                   f"hipEventDisableSystemFence, so no event adds a cache writeback); a {FLUSH_BYTES >> 30} GiB "
                   f"scratch read before every step (outside its events) flushes the caches and leaves them clean; "
                   f"{args.prewarm:g} s of untimed steps and {args.warmup} warm-up steps before the timed ones"
                   if not args.no_flush else "steps timed by HIP events, no cache flush"),
        "roofline": {"bound": "hbm", "kernel": ENTRY[dom], "stage": dom,
                     "achieved": round(stage_rep[dom]["GBps"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(stage_rep[dom]["GBps"] / HBM_PEAK_GBS, 4),
                     "alg_bytes": int(byts[dom]),
                     "traffic": recorded_traffic(ENTRY[dom], cfg.name)},
        "fused_restore_attn": {"GBps": stage_rep["restore_attn"]["GBps"],
                               "frac_hbm_peak": stage_rep["restore_attn"]["frac_hbm_peak"]},
        "collective_reuse_agent_tokens_per_s": agent_tokens / (reuse_ms * 1e-3),
        "stages": stage_rep,
        "per_config": per_config,
        "dense_comparator": main_r["dense"],
        "graph_replay": main_r["graph"],
        "serial_per_agent": main_r["serial"],
        "paged_layout": main_r["paged"],
        "transfer_restore": main_r["transfer"],
        "compression": main_r["compression"],
        "cpu_baseline": None,
    }
    if pool is not None:
        res["cpu_baseline"] = cpu_baseline(pool, n_pool, cfg.name)
        res["gpu_vs_oracle"] = res["value"] / res["cpu_baseline"]["value"]
        for nm, pc in per_config.items():
            if nm == cfg.name:
                pc["cpu_oracle"] = {f: res["cpu_baseline"][f] for f in ("value", "cores", "round_s")}
            elif not args.no_per_config_cpu:
                cb = cpu_baseline(pool, n_pool, nm, CPU_SAMPLE_LAYERS.get(nm))
                pc["cpu_oracle"] = {f: cb[f] for f in ("value", "cores", "round_s", "sample")}
            if "cpu_oracle" in pc:
                pc["gpu_vs_oracle"] = pc["agent_tokens_per_s"] / pc["cpu_oracle"]["value"]
        pool.close()
        pool.join()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
