"""The kernel's GEMV work splits against a plain model (CPU).

The kernel gives every workgroup a contiguous, in-order range of a matrix's
row pairs (sizes within one of each other), and every streamer wave of the
workgroup a contiguous range of the workgroup's units (unit = one 512-element
piece column of one row pair).  The streamer split is even, except that a
boundary that would fall inside a row pair which already holds the previous
boundary moves to that pair's end, so that no row pair is summed by more than
two waves (two additions into a zeroed word commute bitwise).  The split code
itself (dec_internal.h) is compiled here for the host with g++ and driven over
every GEMV phase of every supported workload shape and several grid sizes.
The batched kernel instead gives every workgroup whole 16-row groups, the
larger shares to the last workgroups; that split is checked the same way.
"""
import os
import subprocess

import pytest

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "memory_bound_transformer_persistent_amd", "csrc")
STREAMERS = 7


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("splits") / "split_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, os.path.join(HERE, "split_check.cpp"), "-o", exe],
                   check=True)
    return exe


def model_wg(npairs, G, skip, g):
    if g < skip:
        return 0, 0
    n, gg, GG = npairs, g - skip, G - skip
    return n * gg // GG, n * (gg + 1) // GG


def model_streamers(n, npc):
    """Written from the rule: even boundaries, moved to a pair's end where the
    pair already holds the previous boundary."""
    bounds, prev = [], 0
    for k in range(1, STREAMERS + 1):
        b = max(n * k // STREAMERS, prev)
        same_pair = b // npc == prev // npc
        if prev % npc and same_pair and b % npc:
            b = min(n, (prev // npc + 1) * npc)
        bounds.append((prev, b))
        prev = b
    return bounds


def phases(s):
    """(name, row pairs, row length) of every GEMV phase of a shape."""
    q = s.n_heads * s.head_dim
    return [("qkv", 3 * q // 2, s.d_model), ("o", s.d_model // 2, q), ("gu", s.d_ffn, s.d_model),
            ("down", s.d_model // 2, s.d_ffn), ("lm", s.lm_vocab // 2, s.d_model)]


CASES = []
for wl in ("tiny", "dense2b", "lane2b"):
    shape = synth.shape_for(wl)
    for G in (7, 64, 100, 256):
        for name, npairs, K in phases(shape):
            # batch 1 with few heads: the heads' workgroups take no QKV rows
            skip = shape.n_heads if (name == "qkv" and shape.n_heads <= G // 32) else 0
            CASES.append((wl, G, name, npairs, K, skip))


def run(driver, cases):
    inp = "".join(f"{npairs} {K} {G} {skip}\n" for (_, G, _, npairs, K, skip) in cases)
    out = subprocess.run([driver], input=inp, capture_output=True, text=True, check=True).stdout
    blocks, cur = [], []
    for line in out.splitlines():
        if line == "end":
            blocks.append(cur)
            cur = []
        else:
            cur.append([int(x) for x in line.split()])
    return blocks


def test_splits_match_the_model_and_cover_every_unit_once(driver):
    blocks = run(driver, CASES)
    assert len(blocks) == len(CASES)
    for (wl, G, name, npairs, K, skip), rows in zip(CASES, blocks):
        what = f"{wl} grid {G} {name}"
        npc = (K + 511) // 512
        assert len(rows) == G
        covered = 0
        sizes = []
        for g, p0, p1, *su in rows:
            assert (p0, p1) == model_wg(npairs, G, skip, g), what
            assert p0 == covered or p0 == p1, what           # contiguous, in order
            covered = max(covered, p1)
            if g >= skip:
                sizes.append(p1 - p0)
            n = (p1 - p0) * npc
            got = list(zip(su[0::2], su[1::2]))
            assert got == model_streamers(n, npc), (what, g)
            # the streamers tile [0, n) in order
            assert got[0][0] == 0 and got[-1][1] == n and all(a[1] == b[0] for a, b in zip(got, got[1:])), what
            # no row pair has more than two contributing streamers
            contrib = [0] * (p1 - p0)
            for u0, u1 in got:
                for pair in {u // npc for u in range(u0, u1)}:
                    contrib[pair] += 1
            assert max(contrib, default=0) <= 2, (what, g)
        assert covered == npairs, what
        assert max(sizes) - min(sizes) <= 1, what


def model_groups(n, G, g):
    """Batched kernel: contiguous, in order, sizes n // G or one more, the
    larger ones last (the workgroups past the attention pairs)."""
    sizes = [n // G + (1 if k >= G - n % G else 0) for k in range(G)]
    b = sum(sizes[:g])
    return b, b + sizes[g]


def test_batched_group_split(driver):
    """The 16-row groups of every batched GEMV phase (and a few odd counts)
    over several grids: the model above, every group once."""
    counts = set()
    for wl in ("tiny", "dense2b"):
        s = synth.shape_for(wl)
        q = s.n_heads * s.head_dim
        for rows in (3 * q, s.d_model, 2 * s.d_ffn, s.lm_vocab):
            counts.add((rows + 15) // 16)
    counts |= {1, 5, 255, 256, 257, 864}
    cases = [(n, G) for n in sorted(counts) for G in (7, 64, 100, 256)]
    inp = "".join(f"{n} 0 {G} -1\n" for n, G in cases)
    out = subprocess.run([driver], input=inp, capture_output=True, text=True, check=True).stdout
    blocks = [b.strip().splitlines() for b in out.split("end\n")[:-1]]
    assert len(blocks) == len(cases)
    for (n, G), rows in zip(cases, blocks):
        assert len(rows) == G
        prev = 0
        for line in rows:
            g, b, e = (int(x) for x in line.split())
            assert (b, e) == model_groups(n, G, g), (n, G, g)
            assert b == prev
            prev = e
        assert prev == n
    # dense2b at batch 8: the 96 extra gate/up groups go to workgroups 160-255,
    # the ones past the 160 (sequence, head) attention pairs
    assert [model_groups(864, 256, g)[1] - model_groups(864, 256, g)[0] for g in (0, 159, 160, 255)] == [3, 3, 4, 4]
