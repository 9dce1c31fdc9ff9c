"""Decode benchmark: tokens/s per request at batch 1 on one MI355X.

Main line (the metric): the dense2b workload -- a 25-layer dense decoder,
d_model 2560, 20 heads x 128, SwiGLU 6912, vocab 65536, fp16 weights drawn
N(0, 0.02) from fixed seeds; the 128-token random prompt is prefilled, then
the timed region is K greedy decode steps (default 512, positions 128..639),
K dec_step calls with the token fed back on the device.  By default they are
served by the decode server: a resident launch takes each step from a
host-pinned mailbox, so no kernel boundary falls between tokens (the region is
4 segments, each one server launch ended by dec_sync); --mode step launches
the kernel once per token instead.  One step = one pass over every active
weight (the whole hot path).

The same JSON line also carries, each measured in this run on its own handle:
  workloads.lane2b        one lane of an 8-way split (3 heads, FFN 864, an
                          8192-row LM shard): 128-token prompt + 1024 steps
  workloads.dense2b_long  a 3968-token prompt through the matrix prefill,
                          then 128 steps to the 4096 cap
  workloads.dense2b_b8    8 sequences of 256-token prompts, 256 steps together
                          (value = tokens/s of all 8; per request = of each)
  workloads.moe2b         dense2b's attention with a mixture-of-experts MLP:
                          32 experts of width 1728 in FP8 E4M3, top-4 routing
                          inside the resident kernel; 128-token prompt + 512
                          steps (its roofline counts the active experts only)
  workloads.moe2b_mx      the same with MXFP4 experts (E2M1 pairs, an E8M0
                          scale per 32 weights)
  ttft                    time to first token of the 128-token prompt: one
                          position per step (the decode kernel), batched (8
                          positions per step on the matrix-core kernel) and
                          matrix (every position as a row of the products);
                          ttft.long: the 3968-token prompt, batched and matrix,
                          with the matrix prefill's flop rate against the
                          2.5 PFLOP/s fp16 peak
  generate                the main span in one dec_generate launch
  stream_ceiling          a plain 16-byte non-temporal read of 2 GiB
  cpu_baseline            the CPU oracle on a bounded sample of the same steps

Every roofline object prices its kernel against MI355X's 8 TB/s HBM peak with
ALGORITHMIC bytes per step (every weight byte once, one embedding row per
sequence, the KV-cache rows attention reads at that position and the rows it
appends) divided by the average step duration, measured with HIP events on
the kernel's own stream around the region (for a server launch of n steps,
bytes and duration per launch are both n times these).
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
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "memory_bound_transformer_persistent_amd", "csrc", "dec_kernels.hip")
EXTRAS = ("lane2b", "dense2b_long", "dense2b_b8", "moe2b", "moe2b_mx")
SERVE_IDLE_US = 200000   # decode server: a launch ends after 0.2 s without a step


def kernel_hash():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per step from the committed PMC summary of this kernel and
    workload, if it was taken on this kernel source."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_sha") != kernel_hash() or rec.get("workload") != workload:
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: the process's CPU count
        return os.cpu_count() or 1


def cpu_baseline(shape, tensors, prompt, n_steps):
    """The oracle, untouched, on a bounded sample of the main workload's own steps:
    the same 128-token prompt (prefilled untimed with the oracle's matrix form),
    then the first n_steps greedy decode steps at positions 128.. (the oracle's
    greedy tokens, which equal the GPU's up to near-ties), timed."""
    import oracle as O
    n0 = len(prompt)
    if shape.moe:
        lg, K16, V16, _, _ = O.prefill_matrix_moe(shape, tensors, prompt)
        dec = O.OracleMoEDecoder(shape, tensors)
        dec.Kc[:, :, :n0], dec.Vc[:, :, :n0], dec.pos = K16, V16, n0
    else:
        lg, K16, V16, _ = O.prefill_matrix(shape, tensors, prompt)
        dec = O.OracleDecoder(shape, tensors)
        dec.load_cache(K16, V16, n0)
    tok = O.greedy(lg[-1])
    t0 = time.perf_counter()
    for _ in range(n_steps):
        tok = O.greedy(dec.step(tok))
    dt = time.perf_counter() - t0
    return {"value": round(n_steps / dt, 4), "unit": "tokens/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{n_steps} greedy decode steps at positions {n0}..{n0 + n_steps - 1} of the main workload "
                      f"after its {n0}-token prompt (prompt prefilled untimed with the oracle's matrix form); "
                      f"float64 NumPy oracle, {blas_threads()} BLAS threads; {dt:.1f} s"}


class Run:
    """One handle of one workload, timed on its own stream."""

    def __init__(self, B, R, torch, w, tensors, stream, flags=0, debug=0, serve=False):
        self.B, self.R, self.torch, self.w, self.stream = B, R, torch, w, stream
        self.s, self.nb, self.serve = w.shape, w.batch, serve
        import synth
        self.prompt = synth.make_prompt(self.s.vocab, w.prompt_len, batch=self.nb, seed=w.prompt_seed)
        desc = B.ModelDesc.from_shape(self.s, batch=self.nb)
        desc.flags |= flags      # keep the shape's own flags (MXFP4 experts)
        self.dec = B.Decoder(desc, tensors=tensors, device=0, stream=stream.cuda_stream, debug_flags=debug,
                             serve_idle_us=SERVE_IDLE_US if serve else 0)

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def warm(self, steps):
        self.dec.prefill(self.prompt)
        for _ in range(steps):
            self.dec.step(want_tok=False)
        self.dec.sync()
        self.dec.reset()

    def prefill_ms(self):
        """Time to first token: the prompt's prefill, HIP events on the handle's stream."""
        a, b = self.ev(), self.ev()
        self.torch.cuda.synchronize()
        a.record(self.stream)
        self.dec.prefill(self.prompt)
        b.record(self.stream)
        b.synchronize()
        return a.elapsed_time(b)

    def decode(self, K, nseg=4, mode="step"):
        """K steps from the current position; (region ms, per-segment tokens/s).

        A decode-server handle (serve) runs each segment as one server launch:
        its steps are posted, then dec_sync ends the launch before the
        segment's end event, which would otherwise wait behind it."""
        torch, dec = self.torch, self.dec
        nseg = nseg if mode == "step" and K >= 8 else 1
        bounds = [K * j // nseg for j in range(nseg + 1)]
        evs = [self.ev() for _ in range(nseg + 1)]
        torch.cuda.synchronize()
        # events only around the region and its segments: an event between
        # every two launches would add about 5 us per step; the launches run
        # back to back, so the average launch duration is the region over K
        evs[0].record(self.stream)
        if mode == "generate":
            dec.generate(K)
            evs[1].record(self.stream)
        else:
            for j in range(nseg):
                for _ in range(bounds[j], bounds[j + 1]):
                    dec.step(want_tok=False)
                if self.serve:
                    dec.sync()
                evs[j + 1].record(self.stream)
        evs[-1].synchronize()
        dec.sync()
        region = evs[0].elapsed_time(evs[-1])
        segs = [(bounds[j + 1] - bounds[j]) * self.nb / (evs[j].elapsed_time(evs[j + 1]) / 1e3) for j in range(nseg)]
        return region, segs

    def record(self, pos0, K, region_ms, kernel):
        R, s, nb = self.R, self.s, self.nb
        per_launch = R.mean_step_bytes(s, pos0, K, nb)
        avg_s = region_ms / K / 1e3
        achieved = per_launch / avg_s / 1e9
        req = K / (region_ms / 1e3)
        return {
            "tokens_per_s": round(req * nb, 2), "tokens_per_s_per_request": round(req, 2),
            "ms_per_step": round(region_ms / K, 4), "positions": [pos0, pos0 + K - 1], "batch": nb,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": R.MI355X_HBM_PEAK / 1e9,
                         "unit": "GB/s", "frac": round(achieved / (R.MI355X_HBM_PEAK / 1e9), 4),
                         "traffic": read_traffic(kernel, self.w.name),
                         "kernel": kernel, "algorithmic_bytes_per_launch": int(per_launch),
                         "avg_launch_ms": round(avg_s * 1e3, 4)},
            "roofline_tokens_per_s_per_request": round(R.roofline_tokens_per_s(s, pos0, K, nb), 1),
        }

    def close(self):
        self.dec.close()


def kernel_name(w):
    kind = "batch_" if w.batch > 1 else ("moe_" if w.shape.moe else "")
    return f"dec_resident_{kind}hd{w.shape.head_dim}"


def extra_workload(B, R, torch, name, full_tensors, stream, warmup, serve):
    """One of the other configurations, at its own prompt and step count."""
    import synth
    w = synth.workload(name)
    if w.shape.moe:
        tensors = synth.workload_weights(w)      # its own seeded draw: router, expert codes and scales
    else:
        tensors = synth.lane_from_full(w.shape, full_tensors) if w.lane else full_tensors
    mp = name == "dense2b_long"      # the long prompt goes through the matrix prefill
    r = Run(B, R, torch, w, tensors, stream, flags=B.DEC_FLAG_MATRIX_PREFILL if mp else 0, serve=serve)
    try:
        r.warm(warmup)
        pre = r.prefill_ms()
        pos0 = r.dec.position
        region, segs = r.decode(w.steps)
        out = r.record(pos0, w.steps, region, kernel_name(w))
        out["prefill"] = {"tokens": w.prompt_len, "sequences": w.batch, "ms": round(pre, 3),
                          "mode": "matrix, all positions per product" if mp else "one position per step"}
        out["workload"] = f"{w.name}: {w.description}; prompt {w.prompt_len} + {w.steps} greedy steps, batch {w.batch}"
        if w.shape.moe:
            out["active_bytes_per_step"] = int(R.mean_step_bytes(w.shape, pos0, w.steps, w.batch))
        out["segments_tokens_per_s"] = [round(x, 1) for x in segs]
        return out
    finally:
        r.close()


def measure_ttft(B, R, torch, synth, w, tensors, stream):
    """Time to first token of the workload's prompt through every prefill path,
    and of the 3968-token prompt through the two matrix-core paths."""
    def ttft_ms(wl, fl, reps):
        rt = Run(B, R, torch, wl, tensors, stream, flags=fl)
        rt.warm(0)
        times = []
        for _ in range(reps):
            times.append(rt.prefill_ms())
            rt.dec.reset()
        rt.close()
        return min(times)
    ttft = {"tokens": w.prompt_len}
    for key, fl in (("one_position_per_step_ms", 0), ("batched_8_per_step_ms", B.DEC_FLAG_BATCHED_PREFILL),
                    ("matrix_ms", B.DEC_FLAG_MATRIX_PREFILL)):
        ttft[key] = round(ttft_ms(w, fl, 3), 3)
    wl = synth.workload("dense2b_long")
    long_mp = ttft_ms(wl, B.DEC_FLAG_MATRIX_PREFILL, 3)
    fl_long = R.prefill_flops(wl.shape, wl.prompt_len)
    achieved_tf = fl_long / (long_mp / 1e3) / 1e12
    ttft["long"] = {"tokens": wl.prompt_len, "matrix_ms": round(long_mp, 2),
                    "batched_8_per_step_ms": round(ttft_ms(wl, B.DEC_FLAG_BATCHED_PREFILL, 1), 1),
                    "roofline": {"bound": "mfma", "achieved": round(achieved_tf, 1),
                                 "peak": R.MI355X_FP16_PEAK / 1e12, "unit": "TFLOP/s",
                                 "frac": round(achieved_tf * 1e12 / R.MI355X_FP16_PEAK, 4),
                                 "flops": fl_long, "kernels": "whole prefill (products, attention, "
                                                              "norms, rotary, SwiGLU, LM row)"}}
    ttft["matrix_tflops_128"] = round(R.prefill_flops(w.shape, w.prompt_len) / (ttft["matrix_ms"] / 1e3) / 1e12, 1)
    return ttft


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="dense2b", help="main line's workload (the others run only for dense2b)")
    ap.add_argument("--mode", choices=["serve", "step", "generate"], default="serve",
                    help="step: one dec_step launch per token (token fed back on the device); "
                         "serve: dec_step calls served by the resident decode server (one launch per segment); "
                         "generate: all timed steps inside one dec_generate launch")
    ap.add_argument("--cpu-steps", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the main line (profiling runs)")
    ap.add_argument("--multilaunch", action="store_true", help="one kernel launch per phase (comparison)")
    ap.add_argument("--batched-prefill", action="store_true",
                    help="main line: prefill 8 positions per step on the matrix-core kernel; decode is unchanged")
    ap.add_argument("--ttft-only", action="store_true",
                    help="only the time-to-first-token measurements of dense2b (prefill profiling runs)")
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
    if w.name == "tiny" or s.moe:
        full, tensors = None, synth.workload_weights(w)
    else:
        # every other workload uses the 2.3B model's seeded tensors (a lane slices them)
        full = synth.make_weights(synth.shape_for("dense2b"), seed=0)
        tensors = synth.lane_from_full(s, full) if w.lane else full
    print(f"# weights generated in {time.time() - t_gen:.1f} s", file=sys.stderr, flush=True)

    stream = torch.cuda.Stream(device=0)
    if args.ttft_only:
        if w.name != "dense2b":
            sys.exit("--ttft-only measures the dense2b prompts")
        print(json.dumps({"ttft": measure_ttft(B, R, torch, synth, w, tensors, stream)}), flush=True)
        return
    bp = args.batched_prefill and w.batch == 1
    flags = B.DEC_FLAG_BATCHED_PREFILL if bp else 0
    if args.mode == "serve" and args.multilaunch:
        sys.exit("--mode serve is one resident launch; not with --multilaunch")
    r = Run(B, R, torch, w, tensors, stream, flags=flags,
            debug=B.DEC_DEBUG_MULTILAUNCH if args.multilaunch else 0, serve=args.mode == "serve")
    K, nb = args.steps, w.batch
    # warm-up: prefill + W steps, then rewind so the timed steps are the workload's positions
    r.warm(args.warmup)
    prefill_ms = r.prefill_ms()
    pos0 = r.dec.position
    t0 = time.perf_counter()
    region_ms, segs = r.decode(K, mode="generate" if args.mode == "generate" else "step")
    wall = time.perf_counter() - t0
    if args.mode == "generate":
        bytes_per_launch = sum(R.step_bytes(s, pos0 + i, nb).total for i in range(K))
        avg_launch_s = region_ms / 1e3
    else:
        bytes_per_launch = R.mean_step_bytes(s, pos0, K, nb)
        avg_launch_s = region_ms / K / 1e3
    req_tok_s = K / (region_ms / 1e3)          # tokens/s of each sequence
    tok_s = req_tok_s * nb                     # whole-job tokens/s
    achieved = bytes_per_launch / avg_launch_s / 1e9
    peak = R.MI355X_HBM_PEAK / 1e9
    # per step (counted on single-step launches; a server launch streams the same bytes per step)
    traffic = read_traffic(kernel_name(w), w.name) if args.mode != "generate" and not args.multilaunch else None
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
                     "kernel": kernel_name(w),
                     "algorithmic_bytes_per_launch": int(bytes_per_launch),
                     "avg_launch_ms": round(avg_launch_s * 1e3, 4),
                     # a decode-server launch serves several steps: the two
                     # fields above are then per step, and a launch's duration
                     # in a kernel trace is steps_per_launch times avg_launch_ms
                     "steps_per_launch": K if args.mode == "generate" else (K // len(segs) if args.mode == "serve" else 1),
                     "per": "launch" if args.mode != "serve" else "step"},
        "tokens_per_s_per_request": round(req_tok_s, 2),
        "segments_tokens_per_s": None if len(segs) < 2 else {
            "n": len(segs), "steps_each": K // len(segs), "min": round(min(segs), 2),
            "median": round(float(np.median(segs)), 2), "max": round(max(segs), 2)},
        "prefill": {"tokens": w.prompt_len, "sequences": nb, "ms": round(prefill_ms, 3),
                    "mode": "batched, 8 positions per step" if bp else "one position per step"},
        "roofline_tokens_per_s": round(roof_tps * nb, 1),
        "roofline_tokens_per_s_per_request": round(roof_tps, 1),
        "hbm_GBps_per_step": round(R.mean_step_bytes(s, pos0, K, nb) * req_tok_s / 1e9, 1),
        "wall_s": round(wall, 3),
        "context": {"pages_8xMI300X_tokens_per_s": 3000, "pages_8xH200_tokens_per_s": 2100,
                    "note": "2B fp16, batch 1, 8 GPUs each: other hardware, context only"},
    }
    if args.mode != "generate" and not args.multilaunch:
        # the same positions in one dec_generate launch (context: what the
        # dec_step calls cost beyond one launch), after the timed region
        r.dec.reset()
        r.dec.prefill(r.prompt)
        gen_ms, _ = r.decode(K, mode="generate")
        out["generate"] = {"tokens_per_s": round(K * nb / (gen_ms / 1e3), 2), "ms_per_step": round(gen_ms / K, 4),
                           "launches": 1}
    r.close()
    if w.name == "dense2b" and not args.no_extras and not args.multilaunch:
        out["ttft"] = measure_ttft(B, R, torch, synth, w, tensors, stream)
        out["workloads"] = {}
        for name in EXTRAS:
            print(f"# measuring {name}", file=sys.stderr, flush=True)
            out["workloads"][name] = extra_workload(B, R, torch, name, full, stream, 8, args.mode == "serve")
    # the plain-stream read rate of this device, the practical ceiling under the 8 TB/s peak
    ceiling = B.stream_ceiling(1 << 31, 5)
    out["stream_ceiling"] = {"GBps": round(ceiling, 1), "bytes": 1 << 31, "reps": 5, "kernel": "dec_stream_read",
                             "decode_frac": round(achieved / ceiling, 4)}
    if not args.no_cpu_baseline:
        print("# running the CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(s, tensors, r.prompt[0], args.cpu_steps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
