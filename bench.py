#!/usr/bin/env python3
"""Benchmark: canonical fp64 reduce and scans at N = 2^28 on one MI355X.

One step runs every operation of the hot path once, each over its resident
synthetic input:
  reduce          canonical reduce, L = 128, init = 1.0   (N = 2^28 f64)
  scan_bd256      block_dyadic<256> inclusive scan         (N = 2^28 f64)
  scan_bd16       block_dyadic<16> inclusive scan          (N = 2^28 f64)
  scan_pairwise   pairwise inclusive scan                  (N = 2^28 f64)
  scan_ip128      iterated_pairwise<128> inclusive scan    (N = 2^28 f64)
  rows_reduce     16384 rows x 4096, L = 16                (f64)
  rows_scan_bd16  16384 rows x 4096, block_dyadic<16>      (f64)
value = algorithmic bytes of the step / time of the step (GB/s); reduce
reads N*8 bytes, a scan reads and writes N*8 bytes each (value_n2e28: the
same over the N = 2^28 ops alone).  Before timing, every result is checked
bit for bit against the CPU oracle: the full reduce and row reduce, 64 rows
of the row scan in full, and for every scan 24 mid-block prefixes evaluated
from scratch (the witness method of the canonical-scan README: output hash
and mid-block probe values) plus the scan's back element against the GPU
reduce of the same expression; the witness (output SHA-256, probes PASS
count) goes into the JSON line.

The practical ceilings (bw_probe.hip: a streaming read and a streaming copy
with the scans' tile pattern) are measured in the same run and every op is
also reported as a fraction of its ceiling; the two per-op targets of the
workloads, the f64 reduce (>= 80% of peak) and the float block_dyadic<256>
scan (>= 60% of peak), both at N = 2^28, are timed on their own inputs
(median and 90th percentile of 50 calls) under "targets".

Inside the timed steps every op is bracketed by HIP events on the stream it
runs on; the op with the largest mean time is the dominant kernel of the
roofline object.  Its HBM traffic comes from the rocprofv3 FETCH_SIZE /
WRITE_SIZE summary under profiles/ when that summary was taken from the
kernel sources as they are now (their SHA-256 is stored with it), else null.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-check]
       python bench.py --only copy ...   (a 2 GiB device copy: the reference
                                          for scaling the PMC byte counters)
       python bench.py --only ceiling    (the read and copy ceiling probes)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
HOST_AHEAD_SPIN = 20_000_000  # GPU clock cycles spun before a timed region (a few ms)
N_MAIN = 1 << 28
ROWS, COLS = 16384, 4096
PROFILES = os.path.join(ROOT, "profiles")
# sources whose kernels the traffic summaries describe
def kernel_sources_sha256() -> str:
    """SHA-256 over every source of the library (csrc/*.hip, *.hpp, *.cpp in
    name order): the profiles' traffic figures are reported only while it
    still matches the value stored with them."""
    import glob
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "scan_canonical_reduce_amd", "csrc")
    for p in sorted(glob.glob(os.path.join(d, "*.hip")) + glob.glob(os.path.join(d, "*.hpp")) +
                    glob.glob(os.path.join(d, "*.cpp"))):
        if os.path.basename(p) == "bw_probe.hip":  # the benchmark's probe, not the library
            continue
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()


def workload_tag(op: str) -> str:
    return "f64_16384x4096" if op.startswith("rows_") else "f64_n2e28"


def read_traffic(op: str):
    """HBM bytes per call of op from profiles/traffic_<op>_<workload>.txt
    (lines 'key: value'), or None when missing or taken from other kernel
    sources."""
    path = os.path.join(PROFILES, f"traffic_{op}_{workload_tag(op)}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    try:
        return {"fetch_bytes": int(kv["fetch_bytes_scaled"]),
                "write_bytes": int(kv["write_bytes_scaled"]),
                "bytes": int(kv["fetch_bytes_scaled"]) + int(kv["write_bytes_scaled"]),
                "source": os.path.relpath(path, ROOT)}
    except (KeyError, ValueError):
        return None


PROBE_LIB = os.path.join(ROOT, "scan_canonical_reduce_amd", "libcanon_bwprobe.so")
N_PROBES = 24


def mid_block_probes(n: int, k: int = N_PROBES) -> np.ndarray:
    """k prefix positions, each in the middle of one of k equal blocks of the
    output (the README's mid-block probes), as int64."""
    return np.array([((2 * j + 1) * n) // (2 * k) for j in range(k)], dtype=np.int64)


def parallel_values(fn, idx, dtype, threads=8):
    """fn(i) for every index on a few host threads (the oracle's C code runs
    outside the GIL), as an array of dtype."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=threads) as ex:
        vals = list(ex.map(lambda i: fn(int(i)), idx))
    return np.array(vals, dtype=dtype)


def literal_prefixes(oracle, x_np, idx, policy, param, threads=8):
    """oracle.scan_prefix (each prefix evaluated from scratch) at every index."""
    return parallel_values(lambda i: oracle.scan_prefix(x_np, i, policy, param), idx,
                           x_np.dtype, threads)


def hex_bits(a) -> list:
    a = np.asarray(a)
    u = np.uint64 if a.dtype == np.float64 else np.uint32
    w = 16 if a.dtype == np.float64 else 8
    return [f"{int(v):0{w}x}" for v in a.view(u)]


def bits_equal(a, b) -> np.ndarray:
    a = np.asarray(a)
    b = np.asarray(b, dtype=a.dtype)
    u = np.uint64 if a.dtype == np.float64 else np.uint32
    return a.view(u) == b.view(u)


# (vectors per thread, grid (0: one tile per workgroup), unused LDS bytes per
# workgroup capping the workgroups per CU): the probe variants measured
READ_VARIANTS = ((4, 512, 0), (8, 256, 0), (4, 0, 0))
COPY_VARIANTS = ((2, 0, 40 << 10), (1, 0, 0), (4, 0, 32 << 10))


def measure_ceiling(torch, dev, nbytes=N_MAIN * 8, reps=20, warmup=5):
    """Read and copy ceilings (bw_probe.hip) over `nbytes`: for each variant
    the median of `reps` calls bracketed by HIP events on the current stream;
    the best variant of each kind is the ceiling."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    P, S, I, U = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint
    lib.canon_probe_read.argtypes = [P, S, I, U, U, P, P]
    lib.canon_probe_copy.argtypes = [P, P, S, I, U, U, P]
    a = torch.ones(nbytes // 8, dtype=torch.float64, device=dev)
    b = torch.empty_like(a)
    sink = torch.empty(nbytes // (16 * 256) + 1, dtype=torch.int32, device=dev)  # per workgroup
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream

    def rate(fn, moved):
        for _ in range(warmup):
            assert fn() == 0
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        torch.cuda._sleep(HOST_AHEAD_SPIN)
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        return moved / (ms[reps // 2] * 1e-3) / 1e9

    out = {"variants": {}}
    for kind, variants in (("read", READ_VARIANTS), ("copy", COPY_VARIANTS)):
        best = None
        for v, g, sh in variants:
            if kind == "read":
                fn = (lambda v=v, g=g, sh=sh: lib.canon_probe_read(
                    a.data_ptr(), nbytes, v, g, sh, sink.data_ptr(), st))
                r = rate(fn, nbytes)
            else:
                fn = (lambda v=v, g=g, sh=sh: lib.canon_probe_copy(
                    a.data_ptr(), b.data_ptr(), nbytes, v, g, sh, st))
                r = rate(fn, 2 * nbytes)
            label = f"{kind} {v} vectors/thread, " + \
                (f"grid {g}" if g else "one tile per workgroup") + \
                (f", {sh >> 10} KiB LDS per workgroup" if sh else "")
            out["variants"][label] = round(r, 1)
            log(f"[bench] ceiling {label}: {r:.0f} GB/s")
            if best is None or r > best[0]:
                best = (r, label)
        out[f"{kind}_GBps"] = round(best[0], 1)
        out[f"{kind}_variant"] = best[1]
    out["bytes"] = nbytes
    out["probe"] = "scan_canonical_reduce_amd/csrc/bw_probe.hip"
    del a, b, sink
    return out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-check", action="store_true", help="skip the oracle parity gate")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma list of ops to run (profiling)")
    ap.add_argument("--contrast", action="store_true",
                    help="canonical results against torch.sum / torch.cumsum and the left fold")
    ap.add_argument("--configs", action="store_true",
                    help="time every workload config (parity-checked) and print a table")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU (no collectives); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import scan_canonical_reduce_amd as canon
    import synth

    canon.lib()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.configs:
        run_configs(torch, canon, synth, dev)
        return
    if args.contrast:
        run_contrast(torch, canon, synth, dev)
        return

    only = set(args.only.split(",")) if args.only else None
    if only == {"ceiling"}:
        print(json.dumps({"ceiling": measure_ceiling(torch, dev)}), flush=True)
        return
    want_rows = only is None or bool(only & {"rows_reduce", "rows_scan_bd16"})

    # ------------------------------------------------------------ inputs
    t0 = time.time()
    x_np = synth.config_input("reduce_2e28_f64")  # N = 2^28 mixed magnitude, seed 1003
    X_np = synth.config_input("rows_16384x4096") if want_rows else None
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s "
        f"sha256(x)={synth.sha256(x_np)[:16]}"
        + (f" sha256(X)={synth.sha256(X_np)[:16]}" if want_rows else ""))
    x = torch.from_numpy(x_np).to(dev)
    y = torch.empty_like(x)
    r0 = torch.empty((), dtype=torch.float64, device=dev)
    if want_rows:
        X = torch.from_numpy(X_np).to(dev)
        Y = torch.empty_like(X)
        rr = torch.empty(ROWS, dtype=torch.float64, device=dev)

    have_ip = canon.scan_workspace_bytes(N_MAIN, "iterated_pairwise", 128, 8) > 0
    scans = [("scan_bd256", "block_dyadic", 256), ("scan_bd16", "block_dyadic", 16),
             ("scan_pairwise", "pairwise", 0)]
    if have_ip:
        scans.append(("scan_ip128", "iterated_pairwise", 128))
    # one workspace per op, so that every op's error word can be read after
    # the timed steps
    wss = {"reduce": torch.empty(canon.reduce_workspace_bytes(N_MAIN, 128, 8), dtype=torch.uint8,
                                 device=dev)}
    for name, p, q in scans:
        wss[name] = torch.empty(canon.scan_workspace_bytes(N_MAIN, p, q, 8), dtype=torch.uint8,
                                device=dev)

    ops = {}
    ops["reduce"] = (lambda: canon.reduce(x, 128, 1.0, out=r0, ws=wss["reduce"]), N_MAIN * 8)
    for name, p, q in scans:
        ops[name] = ((lambda p=p, q=q, w=wss[name]: canon.scan(x, p, q, out=y, ws=w)),
                     2 * N_MAIN * 8)
    if want_rows:
        ops["rows_reduce"] = (lambda: canon.reduce_rows(X, 16, 0.0, out=rr), ROWS * COLS * 8)
        ops["rows_scan_bd16"] = (lambda: canon.scan_rows(X, "block_dyadic", 16, out=Y),
                                 2 * ROWS * COLS * 8)
    if only is not None:
        if "copy" in only:  # calibration only, never part of the step
            ops["copy"] = (lambda: y.copy_(x), 2 * N_MAIN * 8)
        ops = {k: v for k, v in ops.items() if k in only}

    # ------------------------------------------------------- parity gate
    parity, witness = {}, {}
    if not args.no_check:
        import oracle
        t0 = time.time()
        rng = np.random.default_rng(2024)
        probes = mid_block_probes(N_MAIN)
        for name, (fn, _) in ops.items():
            if name == "copy":
                continue
            fn()
            torch.cuda.synchronize()
            w = {}
            if name == "reduce":
                want = oracle.reduce(x_np, 128, 1.0)
                got = r0.cpu().numpy().reshape(1)
                err = canon.workspace_error(wss[name])
                ok = bool(bits_equal(got, [want]).all()) and err == 0
                w["sha256"] = synth.sha256(got)
                w["error_word"] = int(err)
            elif name == "rows_reduce":
                want = oracle.reduce_rows(X_np, 16, 0.0)
                got = rr.cpu().numpy()
                ok = bool(bits_equal(got, want).all())
                w["sha256"] = synth.sha256(got)
            elif name == "rows_scan_bd16":
                idx = rng.integers(0, ROWS, 64)
                got = Y[torch.from_numpy(idx).to(dev)].cpu().numpy()
                want = oracle.scan_rows(X_np[idx], "block_dyadic", 16)
                ok = bool(bits_equal(got, want).all())
                w["rows_checked"] = 64
                w["sha256"] = synth.sha256(Y.cpu().numpy())
            else:
                _, p, q = [s for s in scans if s[0] == name][0]
                err = canon.workspace_error(wss[name])
                got = y[torch.from_numpy(probes).to(dev)].cpu().numpy()
                want = literal_prefixes(oracle, x_np, probes, p, q)
                hits = bits_equal(got, want)
                # the back element is the reduce of the same expression (a
                # different kernel); every block size here divides 2^28
                L = q if p == "iterated_pairwise" else 1
                back = canon.reduce(x, L, -0.0).cpu().numpy().reshape(1)
                back_ok = bool(bits_equal(y[-1:].cpu().numpy(), back).all())
                ok = err == 0 and bool(hits.all()) and back_ok
                w.update({"sha256": synth.sha256(y.cpu().numpy()), "probes": int(hits.size),
                          "probes_pass": int(hits.sum()), "back_eq_reduce": back_ok,
                          "error_word": int(err)})
            parity[name] = bool(ok)
            w["pass"] = bool(ok)
            witness[name] = w
            log(f"[bench] parity {name}: {'PASS' if ok else 'FAIL'} {w}")
        log(f"[bench] parity gate {time.time() - t0:.1f}s")
        if not all(parity.values()):
            print(json.dumps({"error": "parity gate failed", "parity": parity,
                              "witness": witness}))
            sys.exit(1)

    # ------------------------------------------------------ step timing
    # every op is bracketed by events on the stream it is launched on (the
    # binding launches on torch's current stream)
    stream = torch.cuda.current_stream()
    names = list(ops)

    def step(evs=None):
        for i, name in enumerate(names):
            if evs is not None:
                evs[i][0].record(stream)
            ops[name][0]()
            if evs is not None:
                evs[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    all_evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in names] for _ in range(args.steps)]
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    # a spin kernel ahead of the timed region keeps the GPU busy while the
    # host enqueues the steps, so the region holds GPU time only (no host
    # launch gap before the first op)
    torch.cuda._sleep(HOST_AHEAD_SPIN)
    a.record(stream)
    for k in range(args.steps):
        step(all_evs[k])
    b.record(stream)
    torch.cuda.synchronize()
    total_ms = a.elapsed_time(b)
    ms_step = total_ms / args.steps
    # every bounded wait of the timed steps ended in time (the last call of
    # each op wrote its error word)
    bad = {k: canon.workspace_error(w) for k, w in wss.items() if k in ops}
    bad = {k: v for k, v in bad.items() if v != 0}
    if bad:
        print(json.dumps({"error": "a bounded wait gave up in the timed steps",
                          "error_words": bad}))
        sys.exit(1)
    step_bytes = sum(nb for _, nb in ops.values())
    value = step_bytes / (ms_step * 1e-3) / 1e9

    per_op = {}
    for i, name in enumerate(names):
        ms = sorted(all_evs[k][i][0].elapsed_time(all_evs[k][i][1]) for k in range(args.steps))
        mean = sum(ms) / len(ms)
        nbytes = ops[name][1]
        per_op[name] = {"ms_mean": mean, "ms_median": ms[len(ms) // 2], "ms_min": ms[0],
                        "ms_max": ms[-1], "bytes": nbytes,
                        "GBps": nbytes / (mean * 1e-3) / 1e9,
                        "pct_hbm_peak": 100.0 * nbytes / (mean * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"[bench] {name:15s} mean {mean * 1e3:9.1f} us  "
            f"{per_op[name]['GBps']:8.1f} GB/s  {per_op[name]['pct_hbm_peak']:5.1f}% of peak")

    # the N = 2^28 ops alone (the rows ops are another shape)
    n28 = [k for k in per_op if not k.startswith("rows_") and k != "copy"]
    value_n2e28 = (sum(per_op[k]["bytes"] for k in n28) /
                   (sum(per_op[k]["ms_mean"] for k in n28) * 1e-3) / 1e9) if n28 else None

    # practical ceilings, and every op against its own (read for the
    # reduces, copy for the scans)
    ceiling = measure_ceiling(torch, dev)
    if ceiling:
        for k, v in per_op.items():
            c = ceiling["read_GBps"] if "reduce" in k else ceiling["copy_GBps"]
            v["pct_ceiling"] = 100.0 * v["GBps"] / c

    targets = {} if only is not None else target_ops(torch, canon, synth, dev,
                                                              args.no_check, x, x_np)

    # dominant kernel: the op with the largest mean time in the timed steps
    dom = max(per_op, key=lambda k: per_op[k]["ms_mean"])
    d = per_op[dom]
    traffic = read_traffic(dom)
    roofline = {"bound": "hbm", "achieved": round(d["GBps"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(d["GBps"] / HBM_PEAK_GBS, 4),
                "traffic": traffic["bytes"] if traffic else None, "kernel": dom,
                "algorithmic_bytes": d["bytes"], "us_mean": round(d["ms_mean"] * 1e3, 1)}
    if traffic:
        roofline["traffic_detail"] = traffic

    cpu = None if args.no_cpu_baseline else cpu_baseline(x_np, X_np, have_ip)

    out = {
        "metric": "GB/s and % HBM peak, bit-exact canonical fp64 reduce & scan, N=2^28, 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": "canonical fp64 reduce (L=128, init=1) and scans "
                               "(block_dyadic<256>, block_dyadic<16>, pairwise"
                               + (", iterated_pairwise<128>" if have_ip else "") +
                               ") over N=2^28 mixed-magnitude doubles, plus 16384x4096 "
                               "row reduce (L=16) and row scan (block_dyadic<16>)",
                   "n": N_MAIN, "rows": ROWS, "cols": COLS,
                   "ops": list(ops.keys())},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "value_n2e28": None if value_n2e28 is None else round(value_n2e28, 1),
        "pct_hbm_peak_n2e28": None if value_n2e28 is None else
        round(100.0 * value_n2e28 / HBM_PEAK_GBS, 2),
        "ceiling": ceiling,
        "targets": targets,
        "parity": parity,
        "witness": witness,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in per_op.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def target_ops(torch, canon, synth, dev, no_check, x64, x64_np, reps=50, warmup=5):
    """The two per-op targets of the workloads, each timed on its own input:
    the f64 reduce at N = 2^28 (L = 128, init 1; >= 80% of peak) and the f32
    block_dyadic<256> scan at N = 2^28 (>= 60% of peak).  `reps` calls each
    bracketed by HIP events: median, p10, p90, and the fraction of peak at
    the median and at p90.  The scan is checked first (24 mid-block prefixes
    evaluated from scratch, back element against the GPU reduce)."""
    import oracle
    out = {}
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        torch.cuda._sleep(HOST_AHEAD_SPIN)
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)  # us

    def entry(t, nbytes, goal, ok):
        med, p10, p90 = t[len(t) // 2], t[len(t) // 10], t[(9 * len(t)) // 10]
        frac = nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS
        frac90 = nbytes / (p90 * 1e-6) / 1e9 / HBM_PEAK_GBS
        return {"us_median": round(med, 1), "us_p10": round(p10, 1), "us_p90": round(p90, 1),
                "bytes": nbytes, "frac": round(frac, 4), "frac_at_p90": round(frac90, 4),
                "target_frac": goal, "met_at_median": frac >= goal, "met_at_p90": frac90 >= goal,
                "bit_exact": ok}

    xn = synth.config_input("scan_2e28_f32")
    x = torch.from_numpy(xn).to(dev)
    y = torch.empty_like(x)
    ws = torch.empty(canon.scan_workspace_bytes(xn.size, "block_dyadic", 256, 4),
                     dtype=torch.uint8, device=dev)
    canon.scan(x, "block_dyadic", 256, out=y, ws=ws)
    ok = canon.workspace_error(ws) == 0
    if not no_check:
        idx = mid_block_probes(xn.size)
        got = y[torch.from_numpy(idx).to(dev)].cpu().numpy()
        want = literal_prefixes(oracle, xn, idx, "block_dyadic", 256)
        back = canon.reduce(x, 1, -0.0).cpu().numpy().reshape(1)
        ok = ok and bool(bits_equal(got, want).all()) and \
            bool(bits_equal(y[-1:].cpu().numpy(), back).all())
    t = timed(lambda: canon.scan(x, "block_dyadic", 256, out=y, ws=ws))
    out["scan_bd256_f32_n2e28"] = entry(t, 2 * xn.nbytes, 0.60, ok)
    log(f"[bench] target scan_bd256_f32_n2e28: {out['scan_bd256_f32_n2e28']}")
    del x, y, ws
    xn, x = x64_np, x64  # the step's own N = 2^28 input
    r = torch.empty((), dtype=x.dtype, device=dev)
    ws = torch.empty(canon.reduce_workspace_bytes(xn.size, 128, 8), dtype=torch.uint8, device=dev)
    canon.reduce(x, 128, 1.0, out=r, ws=ws)
    ok = no_check or bool(bits_equal(r.cpu().numpy().reshape(1),
                                     [oracle.reduce(xn, 128, 1.0)]).all())
    t = timed(lambda: canon.reduce(x, 128, 1.0, out=r, ws=ws))
    out["reduce_f64_n2e28"] = entry(t, xn.nbytes, 0.80, ok)
    log(f"[bench] target reduce_f64_n2e28: {out['reduce_f64_n2e28']}")
    return out


SCRUB_BYTES = 512 << 20  # twice the 256 MB Infinity Cache (MALL)


def run_configs(torch, canon, synth, dev, reps=50, warmup=5):
    """Every workload config: each op checked against the oracle (full result
    for reduces and for the 2^20 scans, 32 sampled prefixes evaluated from
    scratch for the large scans, 64 sampled rows for the row ops), then
    `warmup` untimed calls and `reps` calls each bracketed by HIP events on
    the current stream (median, 10th and 90th percentile; GB/s from the
    median), and the mean of `reps` calls issued back to back between two
    events (no event between calls).  The 2^20 inputs
    are also timed with a 512 MiB buffer rewritten before every call, so that
    neither L2 nor the MALL holds them ("MALL scrubbed" rows).  Prints one
    markdown table."""
    import oracle
    stream = torch.cuda.current_stream()
    rows = []
    scrub_buf = []

    def scrub():
        if not scrub_buf:
            scrub_buf.append(torch.empty(SCRUB_BYTES // 4, dtype=torch.float32, device=dev))
        scrub_buf[0].fill_(1.0)

    def timed(fn, scrubbed=False):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        torch.cuda._sleep(HOST_AHEAD_SPIN)
        for r in range(reps):
            if scrubbed:
                scrub()
            ev[2 * r].record(stream)
            fn()
            ev[2 * r + 1].record(stream)
        torch.cuda.synchronize()
        t = sorted(ev[2 * r].elapsed_time(ev[2 * r + 1]) * 1e3 for r in range(reps))  # us
        chain = None
        if not scrubbed:
            torch.cuda._sleep(HOST_AHEAD_SPIN)
            ev[0].record(stream)
            for _ in range(reps):
                fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            chain = ev[0].elapsed_time(ev[1]) / reps * 1e3
        return {"median": t[reps // 2], "p10": t[reps // 10], "p90": t[(9 * reps) // 10],
                "chain": chain}

    def same(got, want):
        got = np.asarray(got)
        want = np.asarray(want, dtype=got.dtype)
        u = np.uint64 if got.dtype == np.float64 else np.uint32
        return bool(np.array_equal(got.view(u), want.view(u)))

    witness = []

    def add(cfg, op, dt, n, nbytes, t, ok, wit=None):
        us = t["median"]
        gbs = nbytes / (us * 1e-6) / 1e9
        rows.append((cfg, op, dt, n, t, gbs, 100.0 * gbs / HBM_PEAK_GBS, n / (us * 1e-6), ok))
        if wit is not None and not cfg.endswith("MALL scrubbed"):
            witness.append((cfg, op, dt, n, wit, ok))
        log(f"[configs] {cfg} {op}: median {us:.1f} us (p10 {t['p10']:.1f}, p90 {t['p90']:.1f}) "
            f"{gbs:.0f} GB/s parity {'PASS' if ok else 'FAIL'}")

    def reduce_cfg(cfg, name, Ls, init, scrubbed=False):
        xn = synth.config_input(name)
        x = torch.from_numpy(xn).to(dev)
        out = torch.empty((), dtype=x.dtype, device=dev)
        for L in Ls:
            ws = torch.empty(max(canon.reduce_workspace_bytes(xn.size, L, xn.itemsize), 1),
                             dtype=torch.uint8, device=dev)
            canon.reduce(x, L, init, out=out, ws=ws)
            got = out.cpu().numpy().reshape(1)
            ok = same(got, [oracle.reduce(xn, L, init)]) and canon.workspace_error(ws) == 0
            wit = {"sha256": synth.sha256(got), "checked": "the result", "values": hex_bits(got)}
            us = timed(lambda: canon.reduce(x, L, init, out=out, ws=ws))
            add(cfg, f"reduce L={L} init={init}", str(xn.dtype), xn.size, xn.nbytes, us, ok, wit)
            if scrubbed:
                us = timed(lambda: canon.reduce(x, L, init, out=out, ws=ws), scrubbed=True)
                add(cfg + " MALL scrubbed", f"reduce L={L} init={init}", str(xn.dtype), xn.size,
                    xn.nbytes, us, ok)

    def scan_cfg(cfg, name, pols, full, scrubbed=False):
        xn = synth.config_input(name)
        x = torch.from_numpy(xn).to(dev)
        y = torch.empty_like(x)
        for pol, q in pols:
            ws = torch.empty(max(canon.scan_workspace_bytes(xn.size, pol, q, xn.itemsize), 1),
                             dtype=torch.uint8, device=dev)
            canon.scan(x, pol, q, out=y, ws=ws)
            ok = canon.workspace_error(ws) == 0
            yn = y.cpu().numpy()
            idx = mid_block_probes(xn.size)
            # the mid-block probes, each evaluated from scratch
            pv = literal_prefixes(oracle, xn, idx, pol, q)
            hits = bits_equal(yn[idx], pv)
            wit = {"sha256": synth.sha256(yn), "probes": int(hits.size),
                   "probes_pass": int(hits.sum()), "values": hex_bits(yn[idx])}
            ok = ok and bool(hits.all())
            if full:
                ok = ok and same(yn, oracle.scan(xn, pol, q))
                wit["checked"] = "every prefix and the probes"
            else:
                wit["checked"] = "the probes and the back element"
            # scan back == reduce under the same expression (GPU reduce)
            L = q if pol == "iterated_pairwise" else 1
            if pol != "block_dyadic" or xn.size % q == 0:
                back = canon.reduce(x, L, -0.0).cpu().numpy().reshape(1)
                ok = ok and same(yn[-1:], back)
            us = timed(lambda: canon.scan(x, pol, q, out=y, ws=ws))
            label = pol if pol == "pairwise" else f"{pol}<{q}>"
            add(cfg, f"scan {label}", str(xn.dtype), xn.size, 2 * xn.nbytes, us, ok, wit)
            if scrubbed:
                us = timed(lambda: canon.scan(x, pol, q, out=y, ws=ws), scrubbed=True)
                add(cfg + " MALL scrubbed", f"scan {label}", str(xn.dtype), xn.size,
                    2 * xn.nbytes, us, ok)

    reduce_cfg("C1", "reduce_1m", (16, 128), 0.0, scrubbed=True)
    scan_cfg("C2", "scan_1m", (("block_dyadic", 256), ("pairwise", 0)), True, scrubbed=True)
    scrub_buf.clear()
    reduce_cfg("C3", "reduce_2e28_f64", (128,), 1.0)
    reduce_cfg("C3", "reduce_2e29_f32", (128,), 1.0)
    Xn = synth.config_input("rows_16384x4096")
    X = torch.from_numpy(Xn).to(dev)
    rr = torch.empty(Xn.shape[0], dtype=X.dtype, device=dev)
    Y = torch.empty_like(X)
    canon.reduce_rows(X, 16, 0.0, out=rr)
    got = rr.cpu().numpy()
    ok = same(got, oracle.reduce_rows(Xn, 16, 0.0))
    sel = mid_block_probes(Xn.shape[0])
    wit = {"sha256": synth.sha256(got), "checked": "every row", "values": hex_bits(got[sel])}
    add("C4", "row reduce L=16", "float64", Xn.size, Xn.nbytes,
        timed(lambda: canon.reduce_rows(X, 16, 0.0, out=rr)), ok, wit)
    canon.scan_rows(X, "block_dyadic", 16, out=Y)
    Yn = Y.cpu().numpy()
    ok = same(Yn, oracle.scan_rows(Xn, "block_dyadic", 16))
    cells = mid_block_probes(Xn.size)
    wit = {"sha256": synth.sha256(Yn), "checked": "every element",
           "values": hex_bits(Yn.reshape(-1)[cells])}
    add("C4", "row scan block_dyadic<16>", "float64", Xn.size, 2 * Xn.nbytes,
        timed(lambda: canon.scan_rows(X, "block_dyadic", 16, out=Y)), ok, wit)
    del X, Y, rr
    scan_cfg("C5", "scan_2e27_f64", (("iterated_pairwise", 128), ("iterated_pairwise", 16),
                                     ("block_dyadic", 16), ("block_dyadic", 256)), False)
    scan_cfg("C5", "scan_2e28_f32", (("block_dyadic", 256),), False)

    def scan_init_cfg(cfg, name, cases):
        """Scans with an initial value on a workload's input: the first, the
        last and 24 mid-block outputs evaluated from scratch."""
        xn = synth.config_input(name)
        x = torch.from_numpy(xn).to(dev)
        y = torch.empty(xn.size + 1, dtype=x.dtype, device=dev)
        for pol, q, kind, init in cases:
            m = xn.size + (1 if kind == "include_initial" else 0)
            ws = torch.empty(max(canon.scan_workspace_bytes(xn.size, pol, q, xn.itemsize), 1),
                             dtype=torch.uint8, device=dev)
            canon.scan_with_init(x, pol, q, kind, init, out=y[:m], ws=ws)
            ok = canon.workspace_error(ws) == 0
            yn = y[:m].cpu().numpy()
            idx = mid_block_probes(m)
            pv = parallel_values(
                lambda k: oracle.scan_with_init_output(xn, k, pol, q, init, kind), idx, xn.dtype)
            hits = bits_equal(yn[idx], pv)
            ends = [0, 1, m - 1]
            ok = ok and bool(hits.all()) and same(yn[ends], [
                oracle.scan_with_init_output(xn, k, pol, q, init, kind) for k in ends])
            wit = {"sha256": synth.sha256(yn), "probes": int(hits.size),
                   "probes_pass": int(hits.sum()), "values": hex_bits(yn[idx]),
                   "checked": "the probes and the first, second and last outputs"}
            us = timed(lambda: canon.scan_with_init(x, pol, q, kind, init, out=y[:m], ws=ws))
            label = pol if pol == "pairwise" else f"{pol}<{q}>"
            add(cfg, f"scan {kind} init={init} {label}", str(xn.dtype), xn.size,
                xn.nbytes + m * xn.itemsize, us, ok, wit)

    scan_init_cfg("C5 with init", "scan_2e27_f64",
                  (("block_dyadic", 16, "exclusive", 1.0),
                   ("block_dyadic", 256, "include_initial", 1.0),
                   ("pairwise", 0, "exclusive", 1.0),
                   ("iterated_pairwise", 128, "exclusive", 1.0),
                   ("block_dyadic", 16, "inclusive", 1.0)))
    scan_init_cfg("C5 with init", "scan_2e28_f32", (("block_dyadic", 256, "exclusive", 1.0),))

    def op_input(name, op):
        """The workload's input for min / max; for products, factors near 1
        drawn with the workload's size and seed (finite products)."""
        c = synth.CONFIGS[name]
        if op != "mul":
            return synth.config_input(name)
        return (1.0 + synth.generate(c["n"], "uniform_pm1", c["seed"]) * 1e-3).astype(c["dtype"])

    def op_cfg(cfg, name, cases):
        """Other operators on a workload's shape: reduces checked in full,
        scans on 34 sampled outputs evaluated from scratch."""
        for op, what, pol, q in cases:
            xn = op_input(name, op)
            x = torch.from_numpy(xn).to(dev)
            if what == "reduce":
                ws = torch.empty(max(canon.reduce_workspace_bytes(xn.size, q, xn.itemsize), 1),
                                 dtype=torch.uint8, device=dev)
                out = torch.empty((), dtype=x.dtype, device=dev)
                canon.reduce_op(x, q, op, 1.0, out=out, ws=ws)
                got = out.cpu().numpy().reshape(1)
                ok = same(got, [oracle.reduce(xn, q, 1.0, op)])
                wit = {"sha256": synth.sha256(got), "checked": "the result",
                       "values": hex_bits(got)}
                us = timed(lambda: canon.reduce_op(x, q, op, 1.0, out=out, ws=ws))
                add(cfg, f"reduce op={op} L={q} init=1.0", str(xn.dtype), xn.size, xn.nbytes, us,
                    ok, wit)
            else:
                y = torch.empty_like(x)
                ws = torch.empty(max(canon.scan_workspace_bytes(xn.size, pol, q, xn.itemsize), 1),
                                 dtype=torch.uint8, device=dev)
                canon.scan_op(x, pol, q, op, out=y, ws=ws)
                ok = canon.workspace_error(ws) == 0
                yn = y.cpu().numpy()
                idx = mid_block_probes(xn.size)
                ident = canon.IDENTITY[op]
                pv = parallel_values(lambda k: oracle.scan_with_init_output(
                    xn, k, pol, q, ident, "inclusive", op), idx, xn.dtype)
                hits = bits_equal(yn[idx], pv)
                ends = [0, 1, xn.size - 1]
                ok = ok and bool(hits.all()) and same(yn[ends], [
                    oracle.scan_with_init_output(xn, k, pol, q, ident, "inclusive", op)
                    for k in ends])
                wit = {"sha256": synth.sha256(yn), "probes": int(hits.size),
                       "probes_pass": int(hits.sum()), "values": hex_bits(yn[idx]),
                       "checked": "the probes and the first, second and last outputs"}
                us = timed(lambda: canon.scan_op(x, pol, q, op, out=y, ws=ws))
                label = pol if pol == "pairwise" else f"{pol}<{q}>"
                add(cfg, f"scan op={op} {label}", str(xn.dtype), xn.size, 2 * xn.nbytes, us, ok,
                    wit)
            del x

    op_cfg("C3 ops", "reduce_2e28_f64", (("mul", "reduce", None, 128), ("min", "reduce", None, 128),
                                         ("max", "reduce", None, 128)))
    op_cfg("C5 ops", "scan_2e27_f64", (("mul", "scan", "block_dyadic", 256),
                                       ("mul", "scan", "pairwise", 0),
                                       ("mul", "scan", "iterated_pairwise", 128),
                                       ("min", "scan", "block_dyadic", 256),
                                       ("max", "scan", "iterated_pairwise", 128)))

    print("| config | op | dtype | N | median us | p10 us | p90 us | back-to-back mean us | "
          "GB/s | % of 8 TB/s | elements/s | bit-exact |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for cfg, op, dt, n, t, gbs, pct, eps, ok in rows:
        chain = "n/a" if t["chain"] is None else f"{t['chain']:.1f}"
        print(f"| {cfg} | {op} | {dt} | {n} | {t['median']:.1f} | {t['p10']:.1f} | "
              f"{t['p90']:.1f} | {chain} | {gbs:.0f} | {pct:.1f} | {eps:.3g} | "
              f"{'yes' if ok else 'NO'} |")
    # the witness of every config row, in the manner of the canonical-scan
    # README's witness runs: the output's SHA-256, the PASS count of the
    # mid-block probes evaluated from scratch, and the probe values' bits
    print()
    print("| config | op | N | output SHA-256 | checked | probes PASS | mid-block values (bits) |")
    print("|---|---|---|---|---|---|---|")
    for cfg, op, dt, n, wit, ok in witness:
        pr = (f"{wit['probes_pass']}/{wit['probes']}" if "probes" in wit else "n/a")
        print(f"| {cfg} | {op} | {n} | {wit['sha256']} | {wit['checked']} | {pr} | "
              f"{' '.join(wit['values'])} |")


def run_contrast(torch, canon, synth, dev, repeats=10):
    """The canonical library next to what a ROCm user reaches for first:
    torch.sum and torch.cumsum (rocPRIM/hipCUB style reductions and scans) on
    the GPU, and the sequential left fold (std::accumulate, oracle) on the
    CPU, on the same inputs.  Counts the scan outputs that differ from the
    canonical ones, checks each side's scan back element against its own
    reduce, and repeats every GPU call to see whether its bits ever change.
    Prints one markdown table."""
    import oracle
    cases = (("scan_1m", "uniform [0,1)"), ("scan_2e27_f64", "mixed magnitude"))
    out = []

    def bits(t):
        a = t.detach().cpu().numpy()
        return a.view(np.uint64 if a.dtype == np.float64 else np.uint32)

    for name, dist in cases:
        xn = synth.config_input(name)
        if xn.size > (1 << 24):
            xn = xn[:1 << 24]  # the left fold and the comparisons stay short
        x = torch.from_numpy(xn).to(dev)
        n = xn.size
        ts = bits(torch.cumsum(x, 0))
        tr = bits(torch.sum(x).reshape(1))
        t_rep = all(np.array_equal(bits(torch.cumsum(x, 0)), ts) and
                    np.array_equal(bits(torch.sum(x).reshape(1)), tr) for _ in range(repeats))
        lf = oracle.left_fold_scan(xn).view(np.uint64)
        for pol, q in (("pairwise", 0), ("block_dyadic", 256), ("iterated_pairwise", 128)):
            cs = bits(canon.scan(x, pol, q))
            L = q if pol == "iterated_pairwise" else 1
            back_ok = pol != "block_dyadic" or n % q == 0
            cr = bits(canon.reduce(x, L, -0.0).reshape(1)) if back_ok else None
            c_rep = all(np.array_equal(bits(canon.scan(x, pol, q)), cs) for _ in range(repeats))
            label = pol if pol == "pairwise" else f"{pol}<{q}>"
            out.append((f"{name} ({dist}, n={n})", label,
                        int(np.count_nonzero(ts != cs)), int(np.count_nonzero(lf != cs)),
                        bool(ts[-1] == tr[0]),
                        None if cr is None else bool(cs[-1] == cr[0]), t_rep, c_rep))
            log(f"[contrast] {out[-1]}")
    print("| input | canonical policy | torch.cumsum elements differing | left-fold prefixes differing"
          " | torch cumsum[-1] == torch.sum | canonical scan[-1] == reduce | torch repeatable"
          " | canonical repeatable |")
    print("|---|---|---|---|---|---|---|---|")
    for r in out:
        print("| " + " | ".join("n/a" if v is None else str(v) for v in r) + " |")


def cpu_baseline(x_np, X_np, have_ip):
    """The oracle (single-threaded C, as it stands) on a bounded sample of the
    same step: reduce and the pairwise / block_dyadic scans over all 2^28
    elements, the iterated_pairwise<128> scan over the first 2^26 (its oracle
    combines 128 lane values per prefix, about 10x slower per element), the
    row ops over all 16384 rows.  value = algorithmic bytes / seconds."""
    import oracle
    # one core, as a single-threaded baseline; the previous affinity comes back afterwards
    allowed = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    core = min(allowed) if allowed else None
    if core is not None:
        os.sched_setaffinity(0, {core})
    try:
        t0 = time.perf_counter()
        nbytes, sample = _cpu_baseline_work(oracle, x_np, X_np, have_ip)
        dt = time.perf_counter() - t0
    finally:
        if core is not None:
            os.sched_setaffinity(0, allowed)
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2), "cpu": host_cpu_model(),
            "pinned_core": core, "host_threads": os.cpu_count()}


def _cpu_baseline_work(oracle, x_np, X_np, have_ip):
    n = x_np.size
    nbytes = 0
    oracle.reduce(x_np, 128, 1.0)
    nbytes += n * 8
    for p, q in (("block_dyadic", 256), ("block_dyadic", 16), ("pairwise", 0)):
        oracle.scan(x_np, p, q)
        nbytes += 2 * n * 8
    sample = "reduce and the block_dyadic<256>, block_dyadic<16> and pairwise scans over all 2^28"
    if have_ip:
        n_ip = 1 << 26
        oracle.scan(x_np[:n_ip], "iterated_pairwise", 128)
        nbytes += 2 * n_ip * 8
        sample += "; iterated_pairwise<128> over the first 2^26"
    if X_np is not None:
        oracle.reduce_rows(X_np, 16, 0.0)
        nbytes += X_np.size * 8
        oracle.scan_rows(X_np, "block_dyadic", 16)
        nbytes += 2 * X_np.size * 8
        sample += "; row reduce and row scan over all 16384 rows"
    return nbytes, sample


def host_cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
