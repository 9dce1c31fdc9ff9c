"""Decode benchmark: tokens/s per request at batch 1 on one MI355X.

Workload (default "dense2b"): a 25-layer dense decoder, d_model 2560, 20 heads
x 128, SwiGLU 6912, vocab 65536, fp16 weights drawn N(0, 0.02) from fixed
seeds; a 128-token random prompt is prefilled, then the timed region is the
512 greedy decode steps at positions 128..639.  One step = one decode token
= one pass over every active weight (the whole hot path).  --workload
dense2b_b8 decodes 8 independent sequences together (256-token prompts):
`value` is then the whole-job tokens/s (8 per step) and
tokens_per_s_per_request the rate each sequence sees.

Prints one JSON line.  The roofline object prices the resident decode kernel
against MI355X's 8 TB/s HBM peak with ALGORITHMIC bytes per launch: every
weight byte once, one embedding row, the KV-cache rows attention reads at
that position and the rows it appends.  stream_ceiling is the measured read
rate of a plain 16-byte non-temporal stream over 2 GiB on the same device
(dec_stream_ceiling) and the decode rate as a fraction of it.  generate is the
same positions decoded in one dec_generate launch (not the metric: it shows
what the per-token launch costs).  The cpu_baseline object times the
CPU oracle (test infrastructure) on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s per request (bs=1) and achieved HBM GB/s vs peak, 1 MI355X"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_dec_resident_dense2b.txt")
KERNEL_SRC = os.path.join(ROOT, "memory_bound_transformer_persistent_amd", "csrc", "dec_kernels.hip")


def kernel_hash():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def read_traffic(workload):
    """HBM bytes per launch from the committed PMC summary, if it was taken on
    this kernel source and this workload."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    rec = {}
    for line in open(PROFILE_TRAFFIC):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_sha") != kernel_hash() or rec.get("workload") != workload:
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(shape, tensors, prompt_len, n_steps):
    """The oracle, untouched, on a bounded sample: a short prompt then n_steps decode steps."""
    import numpy as np
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the process's CPU count
        threads = os.cpu_count() or 1
    prompt = synth.make_prompt(shape.vocab, prompt_len, seed=1)[0]
    lg, K16, V16, _ = O.prefill_matrix(shape, tensors, prompt)
    dec = O.OracleDecoder(shape, tensors)
    dec.load_cache(K16, V16, prompt_len)
    tok = O.greedy(lg[-1])
    t0 = time.perf_counter()
    for _ in range(n_steps):
        tok = O.greedy(dec.step(tok))
    dt = time.perf_counter() - t0
    return {"value": round(n_steps / dt, 4), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_steps} greedy decode steps of the same model after a {prompt_len}-token prompt "
                      f"(float64 NumPy oracle; prompt prefill untimed); {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="dense2b")
    ap.add_argument("--mode", choices=["step", "generate"], default="step",
                    help="step: one dec_step launch per token (token fed back on the device); "
                         "generate: all timed steps inside one dec_generate launch")
    ap.add_argument("--cpu-steps", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--multilaunch", action="store_true", help="one kernel launch per phase (comparison)")
    ap.add_argument("--batched-prefill", action="store_true",
                    help="prefill 8 positions per step on the matrix-core kernel (DEC_FLAG_BATCHED_PREFILL); "
                         "decode is unchanged")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run plain device-to-device copies of BYTES (HBM counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this decode path runs on one GPU; multi-GPU runs are not part of it "
                                   "(data-parallel serving would run one independent replica per GPU)"}))
        sys.exit(2)

    import numpy as np
    import torch
    import synth

    if args.copy_calibration:
        # a plain copy kernel of known size: reads and writes BYTES once per call
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "calls": 3}), flush=True)
        return
    from memory_bound_transformer_persistent_amd import binding as B
    from memory_bound_transformer_persistent_amd import roofline as R

    assert torch.cuda.is_available(), "bench needs a GPU"
    w = synth.workload(args.workload)
    s = w.shape
    if w.prompt_len + max(args.steps, args.warmup) > s.max_ctx:
        sys.exit("prompt + steps exceed the context cap")
    t_gen = time.time()
    tensors = synth.workload_weights(w)
    nb = w.batch
    prompt = synth.make_prompt(s.vocab, w.prompt_len, batch=nb, seed=w.prompt_seed)   # [batch, n]
    print(f"# weights generated in {time.time() - t_gen:.1f} s", file=sys.stderr, flush=True)

    stream = torch.cuda.Stream(device=0)
    flags = B.DEC_DEBUG_MULTILAUNCH if args.multilaunch else 0
    bp = args.batched_prefill and nb == 1
    dec = B.Decoder(B.ModelDesc.from_shape(s, batch=nb, flags=B.DEC_FLAG_BATCHED_PREFILL if bp else 0),
                    tensors=tensors, device=0, stream=stream.cuda_stream,
                    debug_flags=flags)

    # warm-up: prefill + W steps, then rewind so the timed steps are the workload's positions
    dec.prefill(prompt)
    for _ in range(args.warmup):
        dec.step(want_tok=False)
    dec.sync()
    dec.reset()
    # prefill (time to first token), timed on its own: not part of the metric
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    p0.record(stream)
    first_tok, _ = dec.prefill(prompt)
    p1.record(stream)
    p1.synchronize()
    prefill_ms = p0.elapsed_time(p1)
    pos0 = dec.position

    K = args.steps
    torch.cuda.synchronize()
    # HIP events on the decode stream only around the region and at the
    # boundaries of four segments: an event between every two launches would
    # add about 5 us per step.  The launches run back to back, so the average
    # launch duration is the region over K.
    nseg = 4 if args.mode == "step" and K >= 8 else 1
    bounds = [K * j // nseg for j in range(nseg + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nseg + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    if args.mode == "generate":
        toks = dec.generate(K)
        evs[1].record(stream)
    else:
        for j in range(nseg):
            for _ in range(bounds[j], bounds[j + 1]):
                dec.step(want_tok=False)
            evs[j + 1].record(stream)
    evs[-1].synchronize()
    dec.sync()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = evs[0].elapsed_time(evs[-1])
    if args.mode == "generate":
        bytes_per_launch = sum(R.step_bytes(s, pos0 + i, nb).total for i in range(K))
        avg_launch_s = region_ms / 1e3
    else:
        bytes_per_launch = R.mean_step_bytes(s, pos0, K, nb)
        avg_launch_s = region_ms / K / 1e3
    # the rate of each segment (later segments are at longer contexts)
    segs = None
    if nseg > 1:
        seg_tps = [(bounds[j + 1] - bounds[j]) * nb / (evs[j].elapsed_time(evs[j + 1]) / 1e3) for j in range(nseg)]
        segs = {"n": nseg, "steps_each": K // nseg, "min": round(min(seg_tps), 2),
                "median": round(float(np.median(seg_tps)), 2), "max": round(max(seg_tps), 2)}
    req_tok_s = K / (region_ms / 1e3)          # tokens/s of each sequence
    tok_s = req_tok_s * nb                     # whole-job tokens/s
    achieved = bytes_per_launch / avg_launch_s / 1e9
    peak = R.MI355X_HBM_PEAK / 1e9
    traffic = read_traffic(w.name) if args.mode == "step" and not args.multilaunch else None
    roof_tps = R.roofline_tokens_per_s(s, pos0, K, nb)   # per request

    out = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(region_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}; prompt {w.prompt_len} + {K} greedy decode steps, "
                               f"batch {nb}",
                   "batch": nb, "positions": [pos0, pos0 + K - 1], "mode": args.mode,
                   "launch": "one kernel launch per phase" if args.multilaunch else "resident kernel, grid barriers"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": peak, "unit": "GB/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "kernel": f"dec_resident_{'batch_' if nb > 1 else ''}hd{s.head_dim}",
                     "algorithmic_bytes_per_launch": int(bytes_per_launch),
                     "avg_launch_ms": round(avg_launch_s * 1e3, 4)},
        "tokens_per_s_per_request": round(req_tok_s, 2),
        "segments_tokens_per_s": segs,
        "prefill": {"tokens": w.prompt_len, "sequences": nb, "ms": round(prefill_ms, 3),
                    "mode": "batched, 8 positions per step" if bp else "one position per step"},
        "roofline_tokens_per_s": round(roof_tps * nb, 1),
        "roofline_tokens_per_s_per_request": round(roof_tps, 1),
        "hbm_GBps_per_step": round(R.mean_step_bytes(s, pos0, K, nb) * req_tok_s / 1e9, 1),
        "wall_s": round(wall, 3),
        "context": {"pages_8xMI300X_tokens_per_s": 3000, "pages_8xH200_tokens_per_s": 2100,
                    "note": "2B fp16, batch 1, 8 GPUs each: other hardware, context only"},
    }
    if args.mode == "step" and not args.multilaunch:
        # the same positions in one dec_generate launch (context: the step
        # mode's per-launch cost), after the timed region
        dec.reset()
        dec.prefill(prompt)
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        dec.generate(K)
        g1.record(stream)
        g1.synchronize()
        gen_ms = g0.elapsed_time(g1)
        out["generate"] = {"tokens_per_s": round(K * nb / (gen_ms / 1e3), 2), "ms_per_step": round(gen_ms / K, 4),
                           "launches": 1}
    dec.close()
    # the plain-stream read rate of this device, the practical ceiling under the 8 TB/s peak
    ceiling = B.stream_ceiling(1 << 31, 5)
    out["stream_ceiling"] = {"GBps": round(ceiling, 1), "bytes": 1 << 31, "reps": 5, "kernel": "dec_stream_read",
                             "decode_frac": round(achieved / ceiling, 4)}
    if not args.no_cpu_baseline:
        print("# running the CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(s, tensors, 16, args.cpu_steps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
