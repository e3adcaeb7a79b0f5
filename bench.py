"""Benchmark of the CSA2 hot path on one MI355X.

A step = one decode step of a workload: the step's own token written to every owned KV set (FP4
row + indexer key, one launch per set), then every layer in order (Full: scan + select; Reindex;
Reuse: none), each followed by its gather-dequant attention, which also writes that layer's own
window entry for the token.  Inputs are synthetic and already resident in HBM when the timed
region starts.

Prints ONE JSON line.  `value` is decode tokens/s of the batched 64K-context workload
(32 sequences x 65,536 positions, 8 layers F R R R U U U U), timed over K replays of the step
captured in HIP graphs (the host issues one launch per step); the 1M-context workload (8 x 2^20,
20 layers) is reported in the same line under "also".  `kernels` lists the step's timed kernels
(the Full scan, the Reindex scoring and selection, the attention), each timed with HIP events its own
launches record at the kernel's start and end in K eager steps, with its share of the step, its
algorithmic GB/s and its fraction of HBM peak; `roofline` is the entry with the largest share.
`kv_gather` is the attention's cache gathers (72 B per selected FP4 entry, 256 B per bf16 window
entry) per launch over the attention kernel's duration.  `bulk_append` times fp4_kv_append of
2^20 tokens; `stream_ceiling` a plain 1 GiB device copy (torch) and a 1 GiB streaming read (the
library's own read kernel), the rates this HBM delivers in practice.  `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload on the host's cores.  "also" further holds the 1M-context workload in
the pages' storage formats (FP8 window with SWA Bounded Replay, MXFP4 indexer keys, both), the two
prefill chunks (chunk tokens/s, MFMA roofline of the scoring), the single 4K-context sequence and
the ragged mix of 64 sequences.  The 64K workload rotates two device copies of its inputs so that
no step re-reads data a 256 MiB last-level cache could still hold.

  python bench.py [--steps K] [--warmup W] [--workload 1] [--also 2,5,6,7,3,8,0,4] [--no-cpu-baseline]
  python bench.py --mode copy      # plain 1 GiB device copy, for counter calibration
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X
METRIC = "CSA2 decode tokens/s at 64K & 1M ctx; KV gather GB/s vs HBM peak"
DTYPE = "f16/bf16 MFMA, fp32 accumulate"
STORAGE = ("main KV FP4 (E2M1 + E4M3 per 16 ch); indexer keys bf16 (MXFP4 in the mxkeys workloads); "
           "window bf16 (E4M3 in the fp8win workloads); scores, softmax and outputs fp32")
KERNEL_NAMES = {"scan": "k_idx_score_full", "reindex_score": "k_idx_reindex_score",
                "reindex_select": "k_idx_reindex_select", "attend": "k_attend"}
DECODE_MAX_Q = 64   # attention calls of at most this many queries run k_attend_dec (entries split)


def kernel_name(family: str, n_q: int) -> str:
    if family == "attend" and n_q <= DECODE_MAX_Q:
        return "k_attend_dec"
    return KERNEL_NAMES[family]


# sources whose text decides each timed kernel's code, and the compiler flags of the translation
# units that hold it: a committed counter summary is used for `traffic` only while these still
# hash to the value recorded in it
_COMMON = ["compressed_sparse_attention_07_amd/csrc/csa2_device.hpp"]
KERNEL_SOURCES = {
    "scan": ["compressed_sparse_attention_07_amd/csrc/scan_full.hpp",
             "compressed_sparse_attention_07_amd/csrc/scan_common.hpp"] + _COMMON,
    "reindex_score": ["compressed_sparse_attention_07_amd/csrc/reindex_score.hpp",
                      "compressed_sparse_attention_07_amd/csrc/scan_common.hpp"] + _COMMON,
    "reindex_select": ["compressed_sparse_attention_07_amd/csrc/reindex_select.hpp"] + _COMMON,
    "attend": ["compressed_sparse_attention_07_amd/csrc/attend.hip",
               "compressed_sparse_attention_07_amd/csrc/attend_decode.hip",
               "compressed_sparse_attention_07_amd/csrc/attend_common.hpp",
               "compressed_sparse_attention_07_amd/csrc/pack_common.hpp"] + _COMMON,
}
KERNEL_UNITS = {"scan": ["indexer.hip"], "reindex_score": ["indexer.hip"], "reindex_select": ["indexer.hip"],
                "attend": ["attend.hip", "attend_decode.hip"]}


def source_sha(family: str) -> str:
    from compressed_sparse_attention_07_amd import build as B
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[family]:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    for u in KERNEL_UNITS[family]:
        h.update(" ".join(f for f in B.FLAGS + B.EXTRA.get(u, []) if not f.startswith("-I")).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, family: str, workload_name: str):
    """Calibrated HBM bytes per launch of a kernel from the committed counter summary
    profiles/traffic_<kernel>_<workload>.md, if it was taken on the current sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload_name}.md")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            kv[k.strip()] = v.strip().strip("`")
    if kv.get("source_sha256") != source_sha(family):
        return None
    try:
        return float(kv["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


_SLEEP_CYCLES_PER_S = None


def gpu_busy_wait(torch, seconds: float) -> None:
    """Queue a spin kernel of about `seconds` on the current stream (rate calibrated once)."""
    global _SLEEP_CYCLES_PER_S
    if _SLEEP_CYCLES_PER_S is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1 << 22)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_S = (1 << 22) / max(a.elapsed_time(b) / 1e3, 1e-6)
    torch.cuda._sleep(int(min(seconds, 1.0) * _SLEEP_CYCLES_PER_S))


def measure(wid: int, steps: int, warmup: int, keep_host=False, copies=1):
    """Eager pass with every timed kernel recording its own start and end (average durations),
    then the timed region proper: `steps` replays of the step captured in HIP graphs."""
    import torch
    from compressed_sparse_attention_07_amd import workloads as W

    wl = W.WORKLOADS[wid]
    t_setup = time.perf_counter()
    r = W.Runner(wl, keep_host=keep_host, copies=copies)
    setup_s = time.perf_counter() - t_setup
    print(f"[bench] {wl.name}: setup {setup_s:.1f} s, {copies} input cop{'y' if copies == 1 else 'ies'}",
          file=sys.stderr, flush=True)
    t_host = time.perf_counter()
    for _ in range(warmup):
        r.step()
    t_host = (time.perf_counter() - t_host) / max(warmup, 1)  # host time to issue one step (upper bound)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        r.step()
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - t0
    # the same steps again with the timed kernels recording their own start and end; a GPU-side
    # wait in front lets the host issue every step before the GPU starts
    timing = {}
    gpu_busy_wait(torch, 1.5 * steps * t_host + 2e-3)
    for _ in range(steps):
        r.step(timing=timing)
    torch.cuda.synchronize()
    avg_us = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) * 1e3 for k, v in timing.items()}
    per_step = {k: len(v) / steps for k, v in timing.items()}
    # graph replays: the timed region
    graphs = r.capture()
    for k in range(warmup):
        graphs[k % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        graphs[k % len(graphs)].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    del graphs
    tokens_per_step = wl.prefill_chunk or wl.batch
    alg = r.algorithmic_bytes()
    kb = r.kernel_bytes()
    ms_step = elapsed * 1e3 / steps
    res = {
        "workload": wl.name,
        "tokens_per_s": tokens_per_step * steps / elapsed,
        "ms_per_step": ms_step,
        "eager_tokens_per_s": tokens_per_step * steps / eager_s,
        "alg_bytes_per_step": int(sum(alg.values())),
        "alg_gbps_step": sum(alg.values()) / (ms_step / 1e3) / 1e9,
        "input_copies": copies,
    }
    kernels = []
    for k in ("scan", "reindex_score", "reindex_select", "attend"):
        if k not in avg_us:
            continue
        e = {"kernel": kernel_name(k, r.n_q), "family": k, "avg_launch_us": round(avg_us[k], 2),
             "launches_per_step": per_step[k], "share_of_step": round(avg_us[k] * per_step[k] / (ms_step * 1e3), 4)}
        if not wl.prefill_chunk:
            gbps = kb[k] / (avg_us[k] / 1e6) / 1e9
            e.update({"alg_bytes_per_launch": kb[k], "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)})
        kernels.append(e)
    res["kernels"] = kernels
    if "attend" in avg_us and not wl.prefill_chunk:
        g = kb["kv_gather"] / (avg_us["attend"] / 1e6) / 1e9
        res["kv_gather"] = {"gbps": round(g, 1), "frac": round(g / HBM_PEAK_GBPS, 4),
                            "bytes_per_launch": kb["kv_gather"], "avg_launch_us": round(avg_us["attend"], 2)}
    if wl.prefill_chunk:
        # A prefill chunk's per-query key bytes are re-reads of one shared key array (from the
        # caches), not HBM traffic, so no HBM rate is derived from them; its scoring is one dense
        # contraction (all queries x all visible positions x heads x 64) priced against MFMA.
        for k in ("alg_gbps_step", "alg_bytes_per_step"):
            res[k] = None
        res["hbm_note"] = "prefill: MFMA-bound; per-query key bytes are cache re-reads, no HBM rate given"
        flops = 2.0 * 64 * wl.idx_heads * float(r.q_len.sum())
        scan_s = avg_us["scan"] / 1e6
        tflops = flops / scan_s / 1e12
        res["roofline"] = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                           "kernel": "k_idx_prefill_sample + k_idx_prefill_thresh + k_idx_prefill_cand", "alg_flops_per_launch": flops,
                           "avg_launch_us": round(avg_us["scan"], 2)}
    else:
        dom = max(kernels, key=lambda e: e["share_of_step"])
        res["roofline"] = {"bound": "hbm", "achieved": dom["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": dom["frac"], "traffic": read_traffic(dom["kernel"], dom["family"], wl.name),
                           "kernel": dom["kernel"],
                           "share_of_step": dom["share_of_step"], "alg_bytes_per_launch": dom["alg_bytes_per_launch"],
                           "avg_launch_us": dom["avg_launch_us"]}
    res["config"] = {"workload": wl.name, "batch": wl.batch, "context": wl.context, "layers": wl.layers,
                     "top_k": wl.top_k, "pool_blocks": wl.pool_blocks, "window": wl.window,
                     "query_heads": wl.heads, "indexer_heads": wl.idx_heads}
    return r, res


def bulk_append(reps: int = 10) -> dict:
    """fp4_kv_append of 2^20 post-RoPE tokens (128 channels) in one call, timed with events around
    each call; two input copies alternate so no call re-reads a 256 MiB last-level cache."""
    import torch
    from compressed_sparse_attention_07_amd import csa2 as C, synth

    n = 1 << 20
    sig = synth.channel_sigma(4, synth.T_KV_SIGMA, 128, seq=99)
    xs = [torch.from_numpy(synth.kv_bf16(4, synth.T_KV, n, 128, sig, seq=99 + k).view(np.int16))
          .view(torch.bfloat16).cuda() for k in range(2)]
    codes = torch.empty((n, 64), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, 8), dtype=torch.uint8, device="cuda")
    for k in range(2):
        C.fp4_kv_append(xs[k], codes, scales)
    torch.cuda.synchronize()
    ms = []
    for k in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        C.fp4_kv_append(xs[k % 2], codes, scales)
        b.record()
        ms.append((a, b))
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ms])) * 1e3
    nbytes = n * (256 + 72)
    gbps = nbytes / (us / 1e6) / 1e9
    return {"tokens": n, "avg_call_us": round(us, 2), "alg_bytes": nbytes, "gbps": round(gbps, 1),
            "frac": round(gbps / HBM_PEAK_GBPS, 4), "kernel": "k_fp4_pack128",
            "timing": "events recorded around each call on its stream (2 alternating inputs)"}


def stream_ceiling() -> dict:
    """What the HBM delivers to plain streaming kernels in this run, best of 5 each: a 1 GiB device
    copy (torch, read + write) and a 1 GiB streaming read (the library's csa2_stream_read: 16-byte
    loads over the whole chip, timed by the kernel's own events)."""
    import torch
    from compressed_sparse_attention_07_amd import csa2 as C
    nbytes = 1 << 30
    x = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    sink = torch.empty(C.lib().csa2_stream_read_groups(), dtype=torch.int32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record()

    def copy():
        ev[0].record()
        y.copy_(x)
        ev[1].record()

    def read():
        C.csa2_stream_read(x, sink, ev[0], ev[1])

    out = {}
    for name, fn, moved in (("copy", copy, 2 * nbytes), ("read", read, nbytes)):
        fn()
        torch.cuda.synchronize()
        best = 1e9
        for _ in range(5):
            fn()
            torch.cuda.synchronize()
            best = min(best, ev[0].elapsed_time(ev[1]) / 1e3)
        out[f"{name}_gbps"] = round(moved / best / 1e9, 1)
    out["frac_of_peak"] = {k: round(v / HBM_PEAK_GBPS, 4) for k, v in out.items()}
    del x, y, sink
    torch.cuda.empty_cache()
    return out


def _oracle_step(O, r, i, caches, select_only=False):
    """The oracle's decode step for sequence i.  Returns the rows each owned set attends."""
    wl, h = r.wl, r.host
    r0, n = int(r.q_row0[i]), int(r.q_len[i])
    used = [set() for _ in r.sets]
    for s in range(len(r.sets)):
        O.fp4_quantize(h["x"][s][h["new_rows"][s][i]][None])
    cur, idx, pool = -1, None, None
    for l, m in enumerate(wl.layers):
        if m == "F":
            cur += 1
            idx, p = O.index_full(h["q_idx"][l][i], h["w"][l][i], h["k_idx"][cur][r0:r0 + n], n, wl.top_k, 8,
                                  wl.pool_blocks if pool is None else 0)
            pool = p if pool is None else pool
        elif m == "R":
            idx = O.index_reindex(h["q_idx"][l][i], h["w"][l][i], h["k_idx"][cur][r0:r0 + n], n, pool, wl.top_k, 8)
        if select_only:
            used[cur].update(int(j) for j in idx if 0 <= j < n)
        else:
            codes, scales = caches[cur][i]
            O.attend(h["q"][l][i], codes, scales, n, idx, h["swa"][l], i * r.swa_cap, r.swa_cap, wl.window, r.scale)
    return used


def cpu_baseline(r, n_seq: int, min_seconds: float = 10.0) -> dict:
    """The CPU oracle, as it stands, on n_seq sequences of the workload's decode step, repeated
    until at least min_seconds of wall time have been measured.  The sequences are independent:
    one worker thread per host core of this process's affinity set takes them from a pool (BLAS
    held to one thread per worker; numpy releases the interpreter lock in its array kernels, the
    oracle's Python loops do not, so the threads overlap only partly)."""
    import oracle as O
    from threadpoolctl import threadpool_limits

    h = r.host
    workers = max(1, min(len(os.sched_getaffinity(0)), n_seq))
    with threadpool_limits(limits=1):
        # Cache state before the step (exists before a step, so not timed): the oracle's own
        # quantisation of the rows this step attends, found by an untimed selection pass.
        caches = [[None] * n_seq for _ in r.sets]

        def prepare(i):
            r0, n = int(r.q_row0[i]), int(r.q_len[i])
            used = _oracle_step(O, r, i, None, select_only=True)
            for s in range(len(r.sets)):
                rows = np.array(sorted(used[s]), dtype=np.int64)
                codes = np.zeros((n, 64), dtype=np.uint8)
                scales = np.zeros((n, 8), dtype=np.uint8)
                if rows.size:
                    codes[rows], scales[rows] = O.fp4_quantize(h["x"][s][r0 + rows])
                caches[s][i] = (codes, scales)

        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(prepare, range(n_seq)))
            reps, t = 0, 0.0
            while t < min_seconds:
                t0 = time.perf_counter()
                list(ex.map(lambda i: _oracle_step(O, r, i, caches), range(n_seq)))
                t += time.perf_counter() - t0
                reps += 1
    return {"value": reps * n_seq / t, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{reps} x the decode step of {n_seq} of {r.wl.batch} sequences of {r.wl.name} "
                      f"(all {len(r.wl.layers)} layers), {t:.1f} s wall on {workers} worker threads "
                      f"(one per core of the affinity set)"}


def copy_mode(nbytes: int = 1 << 30, reps: int = 5) -> None:
    import torch
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"mode": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "gbps_read_plus_write": 2 * nbytes / dt / 1e9}))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=1)
    ap.add_argument("--also", type=str, default="2,5,6,7,3,8,0,4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the bulk append and streaming ceilings")
    ap.add_argument("--cpu-seqs", type=int, default=32)
    ap.add_argument("--mode", choices=["bench", "copy"], default="bench")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              f"(multi-GPU sharding is a design note only)", file=sys.stderr)
        return 2
    if args.mode == "copy":
        copy_mode()
        return 0

    import torch
    from compressed_sparse_attention_07_amd import csa2
    csa2.lib()  # fail loudly if the HIP library is missing

    # a working set that could sit in the 256 MiB last-level cache is rotated over two copies
    copies = 2 if args.workload in (0, 1) else 1
    r, main_res = measure(args.workload, args.steps, args.warmup, keep_host=not args.no_cpu_baseline,
                          copies=copies)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(r, min(args.cpu_seqs, r.wl.batch))
        print(f"[bench] cpu baseline: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads", file=sys.stderr,
              flush=True)
    del r
    torch.cuda.empty_cache()
    extras = {}
    if not args.no_extras:
        extras["bulk_append"] = bulk_append()
        extras["stream_ceiling"] = stream_ceiling()
        print(f"[bench] bulk append {extras['bulk_append']['gbps']} GB/s, ceiling {extras['stream_ceiling']}",
              file=sys.stderr, flush=True)
    also = []
    for w in [int(x) for x in args.also.split(",") if x.strip()]:
        rr, res = measure(w, max(3, args.steps // 2), args.warmup, copies=2 if w in (0, 1) else 1)
        del rr
        torch.cuda.empty_cache()
        res["step_frac_of_hbm_peak"] = (round(res["alg_gbps_step"] / HBM_PEAK_GBPS, 4)
                                        if res["alg_gbps_step"] is not None else None)
        also.append(res)
        print(f"[bench] {res['workload']}: {res['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(main_res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "storage": STORAGE,
        "data": "synthetic",
        "config": main_res["config"],
        "roofline": main_res["roofline"],
        "kernels": main_res["kernels"],
        "kv_gather": main_res.get("kv_gather"),
        "step_alg_gbps": (round(main_res["alg_gbps_step"], 1) if main_res["alg_gbps_step"] is not None else None),
        "step_frac_of_hbm_peak": (round(main_res["alg_gbps_step"] / HBM_PEAK_GBPS, 4)
                                  if main_res["alg_gbps_step"] is not None else None),
        "eager_tokens_per_s": round(main_res["eager_tokens_per_s"], 1),
        "input_copies": main_res["input_copies"],
        "timing": "value: K replays of the step captured in HIP graphs; kernels and roofline: HIP events that "
                  "each timed kernel's own launch records at its start and end (csa2_timing.h), in K eager "
                  "steps issued behind a GPU-side wait",
        **extras,
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
