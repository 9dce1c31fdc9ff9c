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
