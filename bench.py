#!/usr/bin/env python3
"""Benchmark of the DCA hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * DCA causal prefill of the Llama2-70B-shaped 32k workload (B 1, 64 query /
    8 KV heads, D 128, L 32768, c 4096, w 1024) = prepare (cos/sin table, key
    rotation, V transpose) + the fused attention kernel, and
  * DCA decode of 16 sequences against a 100001-token cache (64/8 heads, D 128).
Inputs are generated once (seeded, synthetic) and are resident in HBM before
the timed region.  Timing uses HIP events recorded on the stream the library
launches on (torch's current stream).

Printed JSON (one line, stdout):
  value        prefill TFLOP/s at 32k = algorithmic FLOPs / (prepare + attend)
  ms_per_step  wall time of one step (prefill + decode), timed region / K
  roofline     the attention kernel against the bf16 dense MFMA peak
  decode       decode GB/s against the HBM peak
  rope_remap_100k  dca_rope_remap building the decode_100k key cache (GB/s)
  prefill_16k_7b   the DCA prefill of the Llama2-7B-shaped 16k workload (32/32 heads)
  prefill_128k the same prefill at 131072 tokens
  cpu_baseline the fp64 oracle timed on a bounded sample of rows on the host,
               with whole oracle calls beside it (`full_oracle`: the tiny fp32
               prefill, one decode_100k sequence)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DCA prefill TFLOP/s (% bf16 MFMA peak) at 32k/128k; decode GB/s (% HBM)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_llama2_70b_32k_decode_100k.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_flops(B, L, Hq, D):
    """One QK^T and one PV multiply-add per causal pair (diagonal included)."""
    return 4.0 * B * Hq * D * L * (L + 1) / 2.0


def decode_bytes(B, kv_len, Hq, Hkv, D, esize=2):
    """K and V caches read once, plus q in and o out."""
    return B * kv_len * Hkv * D * esize * 2 + 2 * B * Hq * D * esize


def source_hash(files):
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(key):
    """HBM bytes per launch of kernel `key` ("prefill_attend", "prefill_prepare",
    "decode_split", "rope_remap", "prefill_attend_16k" or "prefill_prepare_16k")
    from the committed rocprofv3 counter runs, or None when that kernel's
    source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[key]
        if t["source_sha256"] != source_hash(t["sources"]):
            return None
        return t["bytes_per_launch"]
    except (OSError, ValueError, KeyError, TypeError):
        return None


class ClockSampler:
    """Samples the GPU's current shader clock (the starred line of the
    device's sysfs pp_dpm_sclk) from a background thread while a region runs.
    Reports nothing when the file cannot be read."""

    def __init__(self, dev, period_s=0.002):
        self.path, self.power_path, self.samples, self.power, self.period = None, None, [], [], period_s
        self._stop, self._thread = threading.Event(), None
        try:
            import torch
            p = torch.cuda.get_device_properties(dev)
            base = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
            if os.access(base + "/pp_dpm_sclk", os.R_OK):
                self.path = base + "/pp_dpm_sclk"
            for hw in sorted(os.listdir(base + "/hwmon")):
                f = os.path.join(base, "hwmon", hw, "power1_input")
                if os.access(f, os.R_OK):
                    self.power_path = f
                    break
        except Exception:   # no device properties or no sysfs: report no clock
            pass

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if "*" in line:
                    m = re.search(r"(\d+)\s*mhz", line, re.I)
                    return int(m.group(1)) if m else None
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
            except (OSError, ValueError):
                return
            if v:
                self.samples.append(v)
            if self.power_path:
                try:
                    with open(self.power_path) as f:
                        self.power.append(int(f.read().strip()) / 1e6)   # microwatts
                except (OSError, ValueError):
                    self.power_path = None
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join()

    def summary(self):
        """Statistics over the second half of the samples (the readings are
        averages that trail a change of load)."""
        if not self.samples:
            return None
        v = sorted(self.samples[len(self.samples) // 2:])
        pw = sorted(self.power[len(self.power) // 2:])
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1], "samples": len(v),
                "power_w_median": pw[len(pw) // 2] if pw else None,
                "source": "sysfs pp_dpm_sclk and hwmon power1_input, sampled during extra untimed attention calls"}


def prefill_kernel_name(c, w, D):
    """The attention kernel the library launches for bf16 (chunk size s = c - w):
    the DCA map (1) when s is a multiple of 64, else the split map (3)."""
    s = c - w
    if s % 64 == 0:
        return f"prefill_bf16_pp_kernel<{D}, 0, {2 if s % 128 == 0 else 1}>"
    return f"prefill_bf16_pp_kernel<{D}, 3, {2 if s >= 256 else 1}>"


def cpu_baseline(q, k, v, cfg, seconds):
    """The oracle as it stands, on seeded random rows of one head, for ~`seconds`."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    L, D = cfg["L"], cfg["D"]
    rng = np.random.default_rng(0)
    rows = rng.integers(0, L, size=4096)
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    while done < len(rows):
        batch = rows[done:done + 32]
        oracle.dca_prefill_ref(q, k, v, cfg["c"], cfg["w"], cfg["base"], rows=batch, heads=[0])
        flops += sum(4.0 * D * (int(i) + 1) for i in batch)
        done += len(batch)
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{done} seeded random query rows of head 0 of the llama2_70b_32k prefill "
                      f"(fp64 NumPy form A), {dt:.1f} s; host cores available "
                      f"{len(os.sched_getaffinity(0))}"}


def cpu_full_oracle(dec_one):
    """Whole oracle calls, labelled: the tiny fp32 prefill (every row and
    head) and, when `dec_one` holds it, one decode_100k sequence (q, raw K and
    V of sequence 0)."""
    import oracle
    from long_context_attention_dca_amd import inputs
    out = []
    T = inputs.WORKLOADS["tiny_f32"]
    q, k, v = inputs.prefill_inputs(T["B"], T["L"], T["Hq"], T["Hkv"], T["D"], "fp32", T["seed"])
    t0 = time.perf_counter()
    oracle.dca_prefill_ref(q, k, v, T["c"], T["w"], T["base"])
    dt = time.perf_counter() - t0
    out.append({"label": f"tiny_f32 whole prefill (B {T['B']}, L {T['L']}, Hq {T['Hq']}, D {T['D']}, every row)",
                "seconds": dt, "value": prefill_flops(T["B"], T["L"], T["Hq"], T["D"]) / dt / 1e9, "unit": "GFLOP/s"})
    if dec_one is not None:
        DC = inputs.WORKLOADS["decode_100k"]
        dq1, dk1, dv1 = dec_one
        t0 = time.perf_counter()
        oracle.dca_decode_ref(dq1, dk1, dv1, DC["c"], DC["w"], DC["base"])
        dt = time.perf_counter() - t0
        out.append({"label": f"decode_100k sequence 0 ({DC['kv_len']} cached keys, {DC['Hq']} query heads)",
                    "seconds": dt, "value": decode_bytes(1, DC["kv_len"], DC["Hq"], DC["Hkv"], DC["D"]) / dt / 1e9,
                    "unit": "GB/s"})
    return out


def first_calls(dev):
    """Per-call times (HIP events) of the decode_100k call and the 32k
    attention in the states where first calls were seen to run slow: a cache
    or workspace just built, a new allocation filled by a copy, the same
    buffers again, after an unrelated 3 GiB write, and after 2 s idle.  One
    JSON line per series, with the shader clock read after each call."""
    import torch
    import long_context_attention_dca_amd as dca
    from long_context_attention_dca_amd import inputs
    clk = ClockSampler(dev)

    def series(label, fn, n):
        ms, mhz = [], []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(round(e0.elapsed_time(e1), 3))
            mhz.append(clk._read() if clk.path else None)
        print(json.dumps({"first_calls": label, "ms": ms, "mhz": mhz}), flush=True)

    DC = inputs.WORKLOADS["decode_100k"]
    dq, dk, dv = (x.to(dev) for x in inputs.decode_inputs(DC["B"], DC["kv_len"], DC["Hq"], DC["Hkv"], DC["D"],
                                                          "bf16", DC["seed"]))
    kc = dca.rope_remap(dk, dca.DCA_MAP_KEY, DC["c"], DC["w"], DC["base"], 0)
    del dk
    ws = torch.empty(dca.decode_workspace_bytes(DC["B"], DC["kv_len"], DC["Hq"], DC["Hkv"], DC["D"], torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    dec = lambda kc_: dca.decode(dq, kc_, dv, DC["c"], DC["w"], DC["base"], workspace=ws)
    torch.cuda.synchronize()
    series("decode_100k, cache just built", lambda: dec(kc), 20)
    kc2 = kc.clone()
    torch.cuda.synchronize()
    series("decode_100k, a new allocation filled by a copy", lambda: dec(kc2), 20)
    series("decode_100k, the first cache again", lambda: dec(kc), 10)
    junk = torch.empty(3 << 30, dtype=torch.uint8, device=dev)
    junk.fill_(1)
    torch.cuda.synchronize()
    series("decode_100k, after an unrelated 3 GiB write", lambda: dec(kc), 10)
    del junk
    time.sleep(2.0)
    series("decode_100k, after 2 s idle", lambda: dec(kc), 10)
    del kc, kc2, dq, dv, ws
    torch.cuda.empty_cache()
    P = inputs.WORKLOADS["llama2_70b_32k"]
    q, k, v = (x.to(dev) for x in inputs.prefill_inputs(P["B"], P["L"], P["Hq"], P["Hkv"], P["D"], "bf16", P["seed"]))
    o = torch.empty_like(q)
    nb = dca.prefill_workspace_bytes(P["B"], P["L"], P["Hkv"], P["D"], P["c"], torch.bfloat16)
    w1, w2 = (torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(2))
    att = lambda ws_: dca.prefill_attend(q, ws_, P["Hkv"], P["c"], P["w"], out=o)
    dca.prefill_prepare(k, v, P["c"], P["w"], P["base"], workspace=w1)
    torch.cuda.synchronize()
    series("llama2_70b_32k attention, workspace just prepared", lambda: att(w1), 10)
    dca.prefill_prepare(k, v, P["c"], P["w"], P["base"], workspace=w2)
    torch.cuda.synchronize()
    series("llama2_70b_32k attention, a second workspace just prepared", lambda: att(w2), 10)
    time.sleep(2.0)
    series("llama2_70b_32k attention, the first workspace after 2 s idle", lambda: att(w1), 8)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-128k", action="store_true", help="skip the 131072-token prefill")
    ap.add_argument("--no-7b", action="store_true", help="skip the Llama2-7B-shaped 16k prefill")
    ap.add_argument("--no-s3096", action="store_true",
                    help="skip the 32k prefill with chunk size 3096 (not a multiple of the key tiles)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-selfextend", action="store_true", help="skip the SelfExtend 32k prefill")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the chunked 32k prefill and the ragged / paged 100k decodes")
    ap.add_argument("--no-coarse-fine", action="store_true", help="skip the coarse / fine map 32k prefill")
    ap.add_argument("--only", choices=["prefill", "decode", "prefill128k", "prefill7b", "prefill_s3096", "selfextend",
                                       "coarsefine"],
                    default=None,
                    help="run one workload only (for profiling)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (calibrates HBM byte counters)")
    ap.add_argument("--first-calls", action="store_true",
                    help="only time decode_100k and 32k attention call by call on fresh allocations, "
                         "after other traffic and after idle (where the slow first calls come from)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import long_context_attention_dca_amd as dca
    from long_context_attention_dca_amd import inputs

    if not os.path.exists(dca.library_path()):
        from long_context_attention_dca_amd import build
        build.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n}), flush=True)
        return

    if args.first_calls:
        first_calls(dev)
        return

    P = inputs.WORKLOADS["llama2_70b_32k"]
    DC = inputs.WORKLOADS["decode_100k"]
    P128 = inputs.WORKLOADS["llama2_70b_128k"]
    run_prefill = args.only in (None, "prefill")
    run_decode = args.only in (None, "decode")
    run_128k = (args.only == "prefill128k") or (args.only is None and not args.no_128k)
    P7 = inputs.WORKLOADS["llama2_7b_16k"]
    run_7b = (args.only == "prefill7b") or (args.only is None and not args.no_7b)
    PS = inputs.WORKLOADS["llama2_70b_32k_s3096"]
    run_s3096 = (args.only == "prefill_s3096") or (args.only is None and not args.no_s3096)
    SE = inputs.WORKLOADS["selfextend_70b_32k"]
    run_se = (args.only == "selfextend") or (args.only is None and not args.no_selfextend)
    CF = inputs.WORKLOADS["coarse_fine_70b_32k"]
    run_cf = (args.only == "coarsefine") or (args.only is None and not args.no_coarse_fine)

    # ---------------- inputs, resident in HBM before timing ----------------
    if run_prefill:
        log("generating llama2_70b_32k inputs")
        q_h, k_h, v_h = inputs.prefill_inputs(P["B"], P["L"], P["Hq"], P["Hkv"], P["D"], "bf16", P["seed"])
        q, k, v = q_h.to(dev), k_h.to(dev), v_h.to(dev)
        o = torch.empty_like(q)
        nbytes = dca.prefill_workspace_bytes(P["B"], P["L"], P["Hkv"], P["D"], P["c"], torch.bfloat16)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        # setup: a prepare and a few attention calls on the fresh buffers
        # (the first calls run slower), untimed
        dca.prefill_prepare(k, v, P["c"], P["w"], P["base"], workspace=ws)
        for _ in range(5):
            dca.prefill_attend(q, ws, P["Hkv"], P["c"], P["w"], out=o)
    if run_decode:
        log("generating decode_100k inputs")
        dq_h, dk_h, dv_h = inputs.decode_inputs(DC["B"], DC["kv_len"], DC["Hq"], DC["Hkv"], DC["D"], "bf16",
                                                DC["seed"])
        dec_one = (dq_h[:1].clone(), dk_h[:1].clone(), dv_h[:1].clone())   # for the CPU baseline
        dq = dq_h.to(dev)
        kraw = dk_h.to(dev)
        if args.no_chunked:
            del dk_h   # (kept for the SelfExtend / coarse-fine decode caches otherwise)
        kc = dca.rope_remap(kraw, dca.DCA_MAP_KEY, DC["c"], DC["w"], DC["base"], 0)
        # the cache build itself (dca_rope_remap at DCA_MAP_KEY), timed on its
        # own after untimed calls (fresh buffers run slower at first)
        for _ in range(10):
            dca.rope_remap(kraw, dca.DCA_MAP_KEY, DC["c"], DC["w"], DC["base"], 0, out=kc)
        torch.cuda.synchronize()
        rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for e in rev:
            e[0].record()
            dca.rope_remap(kraw, dca.DCA_MAP_KEY, DC["c"], DC["w"], DC["base"], 0, out=kc)
            e[1].record()
        torch.cuda.synchronize()
        remap_ms = sum(e[0].elapsed_time(e[1]) for e in rev) / len(rev)
        # context for the remap's rate: a plain device copy of the same bytes
        # (the runtime's copy kernel), timed the same way
        cp_dst = torch.empty_like(kraw)
        for _ in range(10):
            cp_dst.copy_(kraw)
        torch.cuda.synchronize()
        for e in rev:
            e[0].record()
            cp_dst.copy_(kraw)
            e[1].record()
        torch.cuda.synchronize()
        copy_ms = sum(e[0].elapsed_time(e[1]) for e in rev) / len(rev)
        del cp_dst
        del kraw
        vc = dv_h.to(dev)
        del dv_h
        dws = torch.empty(dca.decode_workspace_bytes(DC["B"], DC["kv_len"], DC["Hq"], DC["Hkv"], DC["D"],
                                                     torch.bfloat16), dtype=torch.uint8, device=dev)
        # setup: decode calls on the freshly built caches until they run at
        # their steady speed (the first ~10 calls are slower), untimed
        for _ in range(20):
            dca.decode(dq, kc, vc, DC["c"], DC["w"], DC["base"], workspace=dws)
    torch.cuda.synchronize()

    def prefill_step(q_, k_, v_, o_, ws_, cfg, ev):
        ev[0].record()
        dca.prefill_prepare(k_, v_, cfg["c"], cfg["w"], cfg["base"], workspace=ws_)
        ev[1].record()
        dca.prefill_attend(q_, ws_, cfg["Hkv"], cfg["c"], cfg["w"], out=o_)
        ev[2].record()

    def decode_step(ev):
        ev[0].record()
        out = dca.decode(dq, kc, vc, DC["c"], DC["w"], DC["base"], workspace=dws)
        ev[1].record()
        return out

    def events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    # ---------------- the step: prefill 32k + decode 100k ----------------
    pe = [events(3) for _ in range(args.steps)]
    de = [events(2) for _ in range(args.steps)]
    for _ in range(args.warmup):
        if run_prefill:
            prefill_step(q, k, v, o, ws, P, events(3))
        if run_decode:
            decode_step(events(2))
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        if run_prefill:
            prefill_step(q, k, v, o, ws, P, pe[i])
        if run_decode:
            decode_step(de[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    if run_prefill:
        prep_ms = sum(e[0].elapsed_time(e[1]) for e in pe) / args.steps
        att_ms = sum(e[1].elapsed_time(e[2]) for e in pe) / args.steps
        fl = prefill_flops(P["B"], P["L"], P["Hq"], P["D"])
        result["value"] = fl / ((prep_ms + att_ms) * 1e-3) / 1e12
        result["unit"] = "TFLOP/s"
        achieved = fl / (att_ms * 1e-3) / 1e12
        result["roofline"] = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                              "traffic": measured_traffic("prefill_attend"),
                              "kernel": prefill_kernel_name(P["c"], P["w"], P["D"]),
                              "kernel_ms": att_ms, "flops_per_launch": fl}
        # the shader clock under this load, sampled over extra (untimed) attention
        # calls: the spec peak assumes 2.4 GHz
        with ClockSampler(dev) as clk:
            for _ in range(max(5, int(600.0 / att_ms))):   # about 0.6 s of back-to-back calls
                dca.prefill_attend(q, ws, P["Hkv"], P["c"], P["w"], out=o)
            torch.cuda.synchronize()
        clock = clk.summary()
        result["roofline"]["clock"] = clock
        if clock:
            result["roofline"]["frac_at_clock"] = achieved / (PEAK_BF16_TFLOPS * clock["median_mhz"] / 2400.0)
        att_all = sorted(e[1].elapsed_time(e[2]) for e in pe)
        # the prepare pass reads K and V once and writes the rotated keys and
        # the V tiles once (HBM-bound)
        prep_bytes = 4 * P["B"] * P["L"] * P["Hkv"] * P["D"] * 2
        result["prefill_32k"] = {"ms": prep_ms + att_ms, "prepare_ms": prep_ms, "attend_ms": att_ms,
                                 "attend_ms_median": att_all[len(att_all) // 2], "attend_ms_min": att_all[0],
                                 "tflops": result["value"],
                                 "prepare_gbps": prep_bytes / (prep_ms * 1e-3) / 1e9,
                                 "prepare_frac": prep_bytes / (prep_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                                 "prepare_bytes": prep_bytes, "prepare_traffic": measured_traffic("prefill_prepare")}
        # The same pass called back to back (untimed by the step): per-call time
        # over a series, so the HIP events' own dispatch gaps around a single
        # call weigh 1/20 as much.  Context for prepare_frac, not a replacement.
        nb2b = 20
        for _ in range(3):
            dca.prefill_prepare(k, v, P["c"], P["w"], P["base"], workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(nb2b):
            dca.prefill_prepare(k, v, P["c"], P["w"], P["base"], workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        b2b_ms = e0.elapsed_time(e1) / nb2b
        result["prefill_32k"]["prepare_ms_back_to_back"] = b2b_ms
        result["prefill_32k"]["prepare_frac_back_to_back"] = prep_bytes / (b2b_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS
    if run_decode:
        dec_ms = sum(e[0].elapsed_time(e[1]) for e in de) / args.steps
        nb = decode_bytes(DC["B"], DC["kv_len"], DC["Hq"], DC["Hkv"], DC["D"])
        gbps = nb / (dec_ms * 1e-3) / 1e9
        dec_all = sorted(e[0].elapsed_time(e[1]) for e in de)
        result["decode"] = {"ms": dec_ms, "ms_median": dec_all[len(dec_all) // 2], "ms_min": dec_all[0],
                            "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                            "frac": gbps / PEAK_HBM_GBPS, "bytes_per_call": nb, "bound": "hbm",
                            "traffic": measured_traffic("decode_split")}
        if not run_prefill:
            result["value"], result["unit"] = gbps, "GB/s"
        rb = 2 * DC["B"] * DC["kv_len"] * DC["Hkv"] * DC["D"] * 2   # read and write once
        result["rope_remap_100k"] = {"ms": remap_ms, "achieved": rb / (remap_ms * 1e-3) / 1e9, "unit": "GB/s",
                                     "frac": rb / (remap_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "bytes_per_call": rb,
                                     "bound": "hbm", "traffic": measured_traffic("rope_remap"),
                                     "includes": "the decode_100k key cache built at j mod s",
                                     "device_copy_gbps": rb / (copy_ms * 1e-3) / 1e9}
    cfg = {"workload": "llama2_70b_32k prefill + decode_100k" if run_prefill and run_decode else
           ("llama2_70b_32k prefill" if run_prefill else "decode_100k"),
           "prefill": {k_: P[k_] for k_ in ("B", "L", "Hq", "Hkv", "D", "c", "w")},
           "decode": {k_: DC[k_] for k_ in ("B", "kv_len", "Hq", "Hkv", "D", "c", "w")}}
    result["config"] = cfg

    # ---------------- chunked prefill and ragged decode (reported beside) -------
    if run_prefill and not args.no_chunked:
        # the 32k prompt's last 4096 tokens as one chunk over the 28672-token
        # prefix; the rotated key cache is built untimed, as a serving system
        # would hold it
        pos0 = P["L"] - 4096
        kcache = dca.rope_remap(k, dca.DCA_MAP_KEY, P["c"], P["w"], P["base"])
        qchunk = q[:, pos0:].contiguous()
        cws = torch.empty(dca.prefill_workspace_bytes(P["B"], P["L"], P["Hkv"], P["D"], P["c"], torch.bfloat16),
                          dtype=torch.uint8, device=dev)
        ochunk = torch.empty_like(qchunk)
        chunk_call = lambda: dca.prefill_chunk(qchunk, kcache, v, pos0, P["c"], P["w"], P["base"], out=ochunk,
                                               workspace=cws)
        for _ in range(5):   # untimed: the cache was just built
            chunk_call()
        torch.cuda.synchronize()
        nc = max(1, min(args.steps, 5))
        cev = [events(2) for _ in range(nc)]
        for i in range(nc):
            cev[i][0].record()
            chunk_call()
            cev[i][1].record()
        torch.cuda.synchronize()
        c_ms = sum(e[0].elapsed_time(e[1]) for e in cev) / nc
        pairs = sum(range(pos0 + 1, P["L"] + 1))          # causal pairs of rows pos0 .. L-1
        fl = 4.0 * P["B"] * P["Hq"] * P["D"] * pairs
        result["prefill_chunk_32k"] = {"ms": c_ms, "tflops": fl / (c_ms * 1e-3) / 1e12,
                                       "frac": fl / (c_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                       "pos0": pos0, "rows": 4096, "steps": nc,
                                       "includes": "copy of the 32768 cached keys/values into tiles, attention"}
        del kcache, qchunk, cws, ochunk
    if run_decode and not args.no_chunked:
        kvr = [int(x) for x in np.linspace(DC["kv_len"] // 2, DC["kv_len"], DC["B"])]
        dvws = torch.empty(dca.decode_varlen_workspace_bytes(kvr, DC["Hq"], DC["Hkv"], DC["D"], torch.bfloat16),
                           dtype=torch.uint8, device=dev)
        # Warm-up: right after caches are built or copied, the first ~10 decode
        # calls (about 10 ms) run up to 7 % slower than the steady state
        # (measured); each line below is timed after MAP_WARMUP untimed calls
        # (about 40 ms).
        MAP_WARMUP = 50
        for _ in range(MAP_WARMUP):
            dca.decode_varlen(dq, kc, vc, kvr, DC["c"], DC["w"], DC["base"], workspace=dvws)
        torch.cuda.synchronize()
        nd = max(1, min(args.steps, 10))
        dv = [events(2) for _ in range(nd)]
        for i in range(nd):
            dv[i][0].record()
            dca.decode_varlen(dq, kc, vc, kvr, DC["c"], DC["w"], DC["base"], workspace=dvws)
            dv[i][1].record()
        torch.cuda.synchronize()
        dv_ms = sum(e[0].elapsed_time(e[1]) for e in dv) / nd
        nbv = sum(kvr) * DC["Hkv"] * DC["D"] * 2 * 2 + 2 * DC["B"] * DC["Hq"] * DC["D"] * 2
        result["decode_varlen_100k"] = {"ms": dv_ms, "achieved": nbv / (dv_ms * 1e-3) / 1e9, "unit": "GB/s",
                                        "frac": nbv / (dv_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                                        "kv_len": f"{kvr[0]}..{kvr[-1]} evenly spaced", "bytes_per_call": nbv}
        # the same ragged batch from a paged cache: pages of 16 rows handed out
        # in a seeded random order (the pools are built untimed)
        PG = 16
        nblk = -(-DC["kv_len"] // PG)
        perm = torch.randperm(DC["B"] * nblk, generator=torch.Generator().manual_seed(DC["seed"])).to(dev)
        table = perm.view(DC["B"], nblk).to(torch.int32).contiguous()
        pools = []
        for x in (kc, vc):
            pool = torch.empty(DC["B"] * nblk, PG, DC["Hkv"], DC["D"], dtype=x.dtype, device=dev)
            padded = torch.zeros(DC["B"], nblk * PG, DC["Hkv"], DC["D"], dtype=x.dtype, device=dev)
            padded[:, : DC["kv_len"]] = x
            pool[perm] = padded.view(DC["B"] * nblk, PG, DC["Hkv"], DC["D"])
            del padded
            pools.append(pool)
        paged_call = lambda: dca.decode_paged(dq, pools[0], pools[1], table, kvr, DC["c"], DC["w"], DC["base"],
                                              workspace=dvws)
        for _ in range(MAP_WARMUP):
            paged_call()
        torch.cuda.synchronize()
        pv = [events(2) for _ in range(nd)]
        for i in range(nd):
            pv[i][0].record()
            paged_call()
            pv[i][1].record()
        torch.cuda.synchronize()
        pg_ms = sum(e[0].elapsed_time(e[1]) for e in pv) / nd
        result["decode_paged_100k"] = {"ms": pg_ms, "achieved": nbv / (pg_ms * 1e-3) / 1e9, "unit": "GB/s",
                                       "frac": nbv / (pg_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "page_size": PG,
                                       "kv_len": f"{kvr[0]}..{kvr[-1]} evenly spaced", "bytes_per_call": nbv}
        del pools, table, perm
        torch.cuda.empty_cache()
        # the same ragged batch under the SelfExtend (G 8, W 1024) and the
        # guide's coarse / fine (C 512, 4096 -> 32768) maps: two rotated key
        # caches each, built untimed
        kraw = dk_h.to(dev)
        del dk_h
        plain = dca.rope_remap(kraw, dca.DCA_MAP_PLAIN, 1, 0, DC["base"], 0)
        second = torch.empty_like(plain)
        for key, build, call in (
                ("selfextend_decode_100k",
                 lambda: dca.rope_remap(kraw, dca.DCA_MAP_SE_KEY_GROUPED, 8, 1024, DC["base"], 0),
                 lambda ws: dca.selfextend_decode(dq, plain, second, vc, kvr, 8, 1024, DC["base"], workspace=ws)),
                ("coarse_fine_decode_100k",
                 lambda: dca.coarse_fine_key_remap(kraw, 512, 4096, 32768, DC["base"]),
                 lambda ws: dca.coarse_fine_decode(dq, plain, second, vc, kvr, 512, 4096, 32768, DC["base"],
                                                   workspace=ws))):
            second.copy_(build())
            mbytes = (dca.selfextend_decode_workspace_bytes(kvr, DC["Hq"], DC["Hkv"], DC["D"], 8, 1024, torch.bfloat16)
                      if "selfextend" in key else
                      dca.coarse_fine_decode_workspace_bytes(kvr, DC["Hq"], DC["Hkv"], DC["D"], 512, torch.bfloat16))
            mws = torch.empty(mbytes, dtype=torch.uint8, device=dev)
            for _ in range(MAP_WARMUP):
                call(mws)
            torch.cuda.synchronize()
            mev = [events(2) for _ in range(nd)]
            for i in range(nd):
                mev[i][0].record()
                call(mws)
                mev[i][1].record()
            torch.cuda.synchronize()
            m_ms = sum(e[0].elapsed_time(e[1]) for e in mev) / nd
            result[key] = {"ms": m_ms, "achieved": nbv / (m_ms * 1e-3) / 1e9, "unit": "GB/s",
                           "frac": nbv / (m_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                           "kv_len": f"{kvr[0]}..{kvr[-1]} evenly spaced", "bytes_per_call": nbv,
                           "caches": "plain + " + ("grouped (G 8, W 1024)" if "selfextend" in key
                                                   else "coarse-scaled (C 512, kappa 8)")}
            del mws
        del kraw, plain, second
        torch.cuda.empty_cache()

    # ---------------- SelfExtend 32k prefill (reported beside the step) ---------
    if run_se:
        log("generating selfextend_70b_32k inputs")
        sq_h, sk_h, sv_h = inputs.prefill_inputs(SE["B"], SE["L"], SE["Hq"], SE["Hkv"], SE["D"], "bf16",
                                                 SE["seed"])
        sq, sk, sv = sq_h.to(dev), sk_h.to(dev), sv_h.to(dev)
        del sq_h, sk_h, sv_h
        sws = torch.empty(dca.selfextend_workspace_bytes(SE["B"], SE["L"], SE["Hkv"], SE["D"], SE["group"],
                                                         SE["window"], torch.bfloat16),
                          dtype=torch.uint8, device=dev)
        se_call = lambda: dca.selfextend_prefill(sq, sk, sv, SE["group"], SE["window"], SE["base"],
                                                 workspace=sws)
        for _ in range(max(1, args.warmup)):
            se_call()
        torch.cuda.synchronize()
        nse = max(1, min(args.steps, 5))
        sev = [events(2) for _ in range(nse)]
        for i in range(nse):
            sev[i][0].record()
            se_call()
            sev[i][1].record()
        torch.cuda.synchronize()
        se_ms = sum(e[0].elapsed_time(e[1]) for e in sev) / nse
        fl = prefill_flops(SE["B"], SE["L"], SE["Hq"], SE["D"])
        result["selfextend_32k"] = {"ms": se_ms, "tflops": fl / (se_ms * 1e-3) / 1e12,
                                    "frac": fl / (se_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                    "group": SE["group"], "window": SE["window"], "steps": nse,
                                    "includes": "cos/sin table, both key rotations, V layout, attention"}
        if args.only == "selfextend":
            result["value"], result["unit"] = result["selfextend_32k"]["tflops"], "TFLOP/s"
            result["config"] = {"workload": "selfextend_70b_32k",
                                "prefill": {k_: SE[k_] for k_ in ("B", "L", "Hq", "Hkv", "D", "group",
                                                                  "window")}}
        del sq, sk, sv, sws
        torch.cuda.empty_cache()

    # ---------------- coarse / fine map 32k prefill (reported beside the step) --
    if run_cf:
        log("generating coarse_fine_70b_32k inputs")
        cq_h, ck_h, cv_h = inputs.prefill_inputs(CF["B"], CF["L"], CF["Hq"], CF["Hkv"], CF["D"], "bf16",
                                                 CF["seed"])
        cq, ck, cv = cq_h.to(dev), ck_h.to(dev), cv_h.to(dev)
        del cq_h, ck_h, cv_h
        cws = torch.empty(dca.coarse_fine_workspace_bytes(CF["B"], CF["L"], CF["Hkv"], CF["D"], torch.bfloat16),
                          dtype=torch.uint8, device=dev)
        cf_call = lambda: dca.coarse_fine_prefill(cq, ck, cv, CF["chunk"], CF["train_len"], CF["target_len"],
                                                  CF["base"], workspace=cws)
        for _ in range(max(1, args.warmup)):
            cf_call()
        torch.cuda.synchronize()
        ncf = max(1, min(args.steps, 5))
        cfev = [events(2) for _ in range(ncf)]
        for i in range(ncf):
            cfev[i][0].record()
            cf_call()
            cfev[i][1].record()
        torch.cuda.synchronize()
        cf_ms = sum(e[0].elapsed_time(e[1]) for e in cfev) / ncf
        fl = prefill_flops(CF["B"], CF["L"], CF["Hq"], CF["D"])
        result["coarse_fine_32k"] = {"ms": cf_ms, "tflops": fl / (cf_ms * 1e-3) / 1e12,
                                     "frac": fl / (cf_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                     "chunk": CF["chunk"], "train_len": CF["train_len"],
                                     "target_len": CF["target_len"], "steps": ncf,
                                     "includes": "theta table, both key rotations, V layout, attention"}
        if args.only == "coarsefine":
            result["value"], result["unit"] = result["coarse_fine_32k"]["tflops"], "TFLOP/s"
            result["config"] = {"workload": "coarse_fine_70b_32k",
                                "prefill": {k_: CF[k_] for k_ in ("B", "L", "Hq", "Hkv", "D", "chunk",
                                                                  "train_len", "target_len")}}
        del cq, ck, cv, cws
        torch.cuda.empty_cache()

    # ---------------- Llama2-7B-shaped 16k prefill (reported beside the step) --
    if run_7b:
        log("generating llama2_7b_16k inputs")
        q7h, k7h, v7h = inputs.prefill_inputs(P7["B"], P7["L"], P7["Hq"], P7["Hkv"], P7["D"], "bf16", P7["seed"])
        q7, k7, v7 = q7h.to(dev), k7h.to(dev), v7h.to(dev)
        del q7h, k7h, v7h
        o7 = torch.empty_like(q7)
        ws7 = torch.empty(dca.prefill_workspace_bytes(P7["B"], P7["L"], P7["Hkv"], P7["D"], P7["c"],
                                                      torch.bfloat16), dtype=torch.uint8, device=dev)
        for _ in range(max(10, args.warmup)):   # fresh buffers run slower at first
            prefill_step(q7, k7, v7, o7, ws7, P7, events(3))
        torch.cuda.synchronize()
        n7 = max(1, args.steps)
        ev7 = [events(3) for _ in range(n7)]
        for i in range(n7):
            prefill_step(q7, k7, v7, o7, ws7, P7, ev7[i])
        torch.cuda.synchronize()
        prep = sum(e[0].elapsed_time(e[1]) for e in ev7) / n7
        att = sum(e[1].elapsed_time(e[2]) for e in ev7) / n7
        fl = prefill_flops(P7["B"], P7["L"], P7["Hq"], P7["D"])
        result["prefill_16k_7b"] = {"ms": prep + att, "prepare_ms": prep, "attend_ms": att,
                                    "tflops": fl / ((prep + att) * 1e-3) / 1e12,
                                    "attend_tflops": fl / (att * 1e-3) / 1e12,
                                    "frac": fl / (att * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "steps": n7,
                                    "traffic": measured_traffic("prefill_attend_16k"),
                                    "prepare_traffic": measured_traffic("prefill_prepare_16k"),
                                    "shape": {k_: P7[k_] for k_ in ("B", "L", "Hq", "Hkv", "D", "c", "w")}}
        if args.only == "prefill7b":
            result["value"], result["unit"] = result["prefill_16k_7b"]["tflops"], "TFLOP/s"
            result["config"] = {"workload": "llama2_7b_16k prefill",
                                "prefill": {k_: P7[k_] for k_ in ("B", "L", "Hq", "Hkv", "D", "c", "w")}}
        del q7, k7, v7, o7, ws7
        torch.cuda.empty_cache()

    # ---------------- 32k prefill, chunk size 3096 (reported beside the step) --
    if run_s3096:
        log("generating llama2_70b_32k_s3096 inputs")
        qsh, ksh, vsh = inputs.prefill_inputs(PS["B"], PS["L"], PS["Hq"], PS["Hkv"], PS["D"], "bf16", PS["seed"])
        qs, ks, vs = qsh.to(dev), ksh.to(dev), vsh.to(dev)
        del qsh, ksh, vsh
        os_ = torch.empty_like(qs)
        wss = torch.empty(dca.prefill_workspace_bytes(PS["B"], PS["L"], PS["Hkv"], PS["D"], PS["c"],
                                                      torch.bfloat16), dtype=torch.uint8, device=dev)
        for _ in range(max(5, args.warmup)):   # fresh buffers run slower at first
            prefill_step(qs, ks, vs, os_, wss, PS, events(3))
        torch.cuda.synchronize()
        ns = max(1, args.steps)
        evs = [events(3) for _ in range(ns)]
        for i in range(ns):
            prefill_step(qs, ks, vs, os_, wss, PS, evs[i])
        torch.cuda.synchronize()
        prep = sum(e[0].elapsed_time(e[1]) for e in evs) / ns
        att = sum(e[1].elapsed_time(e[2]) for e in evs) / ns
        fl = prefill_flops(PS["B"], PS["L"], PS["Hq"], PS["D"])
        result["prefill_32k_s3096"] = {"ms": prep + att, "prepare_ms": prep, "attend_ms": att,
                                       "tflops": fl / ((prep + att) * 1e-3) / 1e12,
                                       "attend_tflops": fl / (att * 1e-3) / 1e12,
                                       "frac": fl / (att * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "steps": ns,
                                       "kernel": prefill_kernel_name(PS["c"], PS["w"], PS["D"]),
                                       "shape": {k_: PS[k_] for k_ in ("B", "L", "Hq", "Hkv", "D", "c", "w")}}
        if run_prefill:
            result["prefill_32k_s3096"]["vs_aligned_attend"] = att / result["prefill_32k"]["attend_ms"]
        if args.only == "prefill_s3096":
            result["value"], result["unit"] = result["prefill_32k_s3096"]["tflops"], "TFLOP/s"
            result["config"] = {"workload": "llama2_70b_32k_s3096 prefill",
                                "prefill": {k_: PS[k_] for k_ in ("B", "L", "Hq", "Hkv", "D", "c", "w")}}
        del qs, ks, vs, os_, wss
        torch.cuda.empty_cache()

    # ---------------- 128k prefill (reported beside the step) ----------------
    if run_128k:
        if run_prefill:
            del o, ws
        if run_decode:
            del kc, vc, dws
        torch.cuda.empty_cache()
        log("generating llama2_70b_128k inputs")
        q2h, k2h, v2h = inputs.prefill_inputs(P128["B"], P128["L"], P128["Hq"], P128["Hkv"], P128["D"], "bf16",
                                              P128["seed"])
        q2, k2, v2 = q2h.to(dev), k2h.to(dev), v2h.to(dev)
        del q2h, k2h, v2h
        o2 = torch.empty_like(q2)
        ws2 = torch.empty(dca.prefill_workspace_bytes(P128["B"], P128["L"], P128["Hkv"], P128["D"], P128["c"],
                                                      torch.bfloat16), dtype=torch.uint8, device=dev)
        n128 = max(1, min(args.steps, 3))
        prefill_step(q2, k2, v2, o2, ws2, P128, events(3))
        torch.cuda.synchronize()
        ev128 = [events(3) for _ in range(n128)]
        for i in range(n128):
            prefill_step(q2, k2, v2, o2, ws2, P128, ev128[i])
        torch.cuda.synchronize()
        prep = sum(e[0].elapsed_time(e[1]) for e in ev128) / n128
        att = sum(e[1].elapsed_time(e[2]) for e in ev128) / n128
        fl = prefill_flops(P128["B"], P128["L"], P128["Hq"], P128["D"])
        result["prefill_128k"] = {"ms": prep + att, "prepare_ms": prep, "attend_ms": att,
                                  "tflops": fl / ((prep + att) * 1e-3) / 1e12,
                                  "attend_tflops": fl / (att * 1e-3) / 1e12,
                                  "frac": fl / (att * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "steps": n128}
        if args.only == "prefill128k":
            result["value"], result["unit"] = result["prefill_128k"]["tflops"], "TFLOP/s"
            result["config"] = {"workload": "llama2_70b_128k prefill",
                                "prefill": {k_: P128[k_] for k_ in ("B", "L", "Hq", "Hkv", "D", "c", "w")}}

    if run_prefill and not args.no_cpu_baseline:
        log(f"cpu baseline: oracle for ~{args.cpu_seconds:.0f} s")
        result["cpu_baseline"] = cpu_baseline(q_h, k_h, v_h, P, args.cpu_seconds)
        log("cpu baseline: whole oracle calls (tiny fp32 prefill, one decode_100k sequence)")
        result["cpu_baseline"]["full_oracle"] = cpu_full_oracle(dec_one if run_decode else None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
