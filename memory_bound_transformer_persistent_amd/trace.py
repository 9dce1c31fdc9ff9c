"""Summaries of the resident kernel's phase trace (DEC_DEBUG_TRACE).

For every phase j of a launch each workgroup g stores two wall-clock stamps,
start[g, j] (after the barrier released it) and end[g, j] (when it arrived at
the next barrier).  From them:
  work     median over workgroups of end - start (time spent in the phase)
  slowest  max over workgroups of end - start
  barrier  min_g start[g, j+1] - max_g end[g, j]: from the last arrival to the
           first release, i.e. the barrier's own latency
  span     max_g end[g, j] - max_g end[g, j-1]: wall time the phase adds
"""
import numpy as np

PHASES = ("qkv", "attn", "o", "gu", "down")


def phase_names(n_layers, n_tok=1, lm=True):
    names = []
    for _ in range(n_tok):
        for l in range(n_layers):
            names += [f"{p}{l}" for p in PHASES]
        if lm:
            names += ["lm", "argmax"]
    return names


def summarize(stamps, hz, n_layers):
    """Per phase kind: mean over layers of (work, slowest, barrier, span) in microseconds."""
    n_ph = 5 * n_layers + 2
    st = stamps[:, 0:2 * n_ph:2].astype(np.float64)
    en = stamps[:, 1:2 * n_ph:2].astype(np.float64)
    us = 1e6 / hz
    work = np.median(en - st, axis=0) * us
    slow = np.max(en - st, axis=0) * us
    last_end = np.max(en, axis=0)
    barrier = np.zeros(n_ph)
    barrier[1:] = (np.min(st[:, 1:], axis=0) - last_end[:-1]) * us
    span = np.zeros(n_ph)
    span[0] = (last_end[0] - np.min(st[:, 0])) * us
    span[1:] = (last_end[1:] - last_end[:-1]) * us
    names = phase_names(n_layers)
    out = {}
    for kind in PHASES + ("lm", "argmax"):
        idx = [i for i, n in enumerate(names) if n.rstrip("0123456789") == kind]
        out[kind] = dict(work=float(np.mean(work[idx])), slowest=float(np.mean(slow[idx])),
                         barrier=float(np.mean(barrier[idx])), span=float(np.mean(span[idx])), count=len(idx))
    total = (last_end[-1] - np.min(st[:, 0])) * us
    return out, float(total)


def format_summary(out, total):
    lines = [f"{'phase':8s} {'count':>5s} {'work us':>9s} {'slowest':>9s} {'barrier':>9s} {'span us':>9s} {'span total':>11s}"]
    for k, v in out.items():
        lines.append(f"{k:8s} {v['count']:5d} {v['work']:9.2f} {v['slowest']:9.2f} {v['barrier']:9.2f} "
                     f"{v['span']:9.2f} {v['span'] * v['count']:11.1f}")
    lines.append(f"launch total {total:.1f} us")
    return "\n".join(lines)


def main(argv):
    """python -m memory_bound_transformer_persistent_amd.trace [WORKLOAD] [STEPS]

    Per-phase summary of single-step decode launches with DEC_DEBUG_TRACE:
    the workload's prompt is prefilled, then STEPS launches of one token each
    are traced and their summaries averaged (the stamps add a few
    microseconds per launch, so the totals sit slightly above untraced steps).
    """
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import torch
    import synth
    from memory_bound_transformer_persistent_amd import binding as B

    name = argv[0] if argv else "dense2b"
    steps = int(argv[1]) if len(argv) > 1 else 16
    w = synth.workload(name)
    s = w.shape
    tensors = synth.workload_weights(w)
    prompt = synth.make_prompt(s.vocab, w.prompt_len, batch=w.batch, seed=w.prompt_seed)
    stream = torch.cuda.Stream(device=0)
    sums, total = None, 0.0
    with B.Decoder(B.ModelDesc.from_shape(s, batch=w.batch), tensors=tensors, device=0, stream=stream.cuda_stream,
                   debug_flags=B.DEC_DEBUG_TRACE) as dec:
        dec.prefill(prompt)
        for _ in range(4):
            dec.step()
        pos0 = dec.position
        for _ in range(steps):
            dec.step()
            stamps, hz = dec.read_trace()
            out, tot = summarize(stamps, hz, s.n_layers)
            total += tot / steps
            if sums is None:
                sums = {k: dict(v) for k, v in out.items()}
                for v in sums.values():
                    for f in ("work", "slowest", "barrier", "span"):
                        v[f] /= steps
            else:
                for k, v in out.items():
                    for f in ("work", "slowest", "barrier", "span"):
                        sums[k][f] += v[f] / steps
    print(f"{name}: {steps} traced single-step launches at positions {pos0}..{pos0 + steps - 1}, "
          f"batch {w.batch}; per phase kind, mean over layers and launches (us)")
    print(format_summary(sums, total))
    return 0


if __name__ == "__main__":
    import sys
    sys.exit(main(sys.argv[1:]))
