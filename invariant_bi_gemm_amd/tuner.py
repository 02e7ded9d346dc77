"""Offline pin tuner: choose one layer's pin from its shape and a workload profile.

The pin of a layer (N, K) is its reduction tree -- the number S of contiguous
equal K splits -- plus a tiling knob, the row count at or below which calls
run the weight-streaming kernel.  Both are fixed before deployment and never
read the batch (Detent, §3: pins and knobs form a commitment tuple fixed for
a workload; §6: the tuner picks it per workload).

Cost model (Detent, §6 eq. 3, restricted to one kernel family): a workload
profile W = {(M, n)} lists the row counts its calls have and how often; the
cost of a legal assignment a is T(a) = sum over W of n * t(M, a), with t
measured on the device; the tuner returns argmin T.  Candidates are legal by
construction (S divides K into whole 64-wide stages; the library checks it
again); each is measured by creating a handle with the pin swapped in
(Detent, §6 "Search": a repin swaps the constants without solving again).
The grids here are small, so the search is exhaustive.

Usage:
    python -m invariant_bi_gemm_amd.tuner --shape 4096x14336 \
        --profile 1:8,2:8,4:8,8:8,16:8,32:4,64:4,128:2,256:2,512:1,1024:1,2048:1,4096:1,8192:1 \
        --table invariant_bi_gemm_amd/pins/gfx950.txt --write

The table keeps one line per (arch, N, K); writing replaces the shape's line,
keeps the others and bumps the version (a new table version may give
different bits, as a different commitment tuple does).
"""
from __future__ import annotations

import argparse
import os
import sys

SPLIT_CHOICES = (1, 2, 4, 7, 8, 14, 16)
STREAM_CHOICES = (0, 16, 32, 64)
MAX_SPLITS = 16


def parse_profile(text: str):
    """'M:n,M:n,...' -> [(M, n)], M >= 1, n >= 1, M unique."""
    out = []
    seen = set()
    for item in text.split(","):
        item = item.strip()
        if not item:
            continue
        m, _, n = item.partition(":")
        m, n = int(m), int(n or 1)
        if m < 1 or n < 1:
            raise ValueError("profile entries need M >= 1 and a count >= 1: %r" % item)
        if m in seen:
            raise ValueError("M=%d listed twice" % m)
        seen.add(m)
        out.append((m, n))
    if not out:
        raise ValueError("empty profile")
    return out


def legal_splits(k: int, choices=SPLIT_CHOICES):
    """Split counts S that cut K into equal whole 64-wide stages."""
    return [s for s in choices if 1 <= s <= MAX_SPLITS and k % (64 * s) == 0]


def candidates(n: int, k: int, profile, split_choices=SPLIT_CHOICES, stream_choices=STREAM_CHOICES):
    """All legal (splits, stream_max_m) pairs; stream thresholds above the
    profile's largest M are equivalent to it and dropped."""
    mmax = max(m for m, _ in profile)
    sm = sorted({min(v, mmax) for v in stream_choices})
    return [(s, v) for s in legal_splits(k, split_choices) for v in sm]


def cost(profile, timing):
    """Detent eq. 3 for one family: sum of count * time over the profile."""
    return sum(n * timing[m] for m, n in profile)


def choose(profile, measure, cands):
    """argmin over candidates of the profile cost; `measure(cand)` returns
    {M: seconds}.  Ties go to the earlier candidate (fewer splits first)."""
    best = None
    report = []
    for c in cands:
        t = measure(c)
        total = cost(profile, t)
        report.append((c, total, t))
        if best is None or total < best[1]:
            best = (c, total)
    return best[0], report


# --- pin table ---------------------------------------------------------------

def read_table(path: str):
    """-> (version, header comment lines, {(arch, N, K): (splits, stream_max_m)})."""
    version = 0
    header = []
    rows = {}
    if not os.path.exists(path):
        return version, header, rows
    for line in open(path):
        raw = line.rstrip("\n")
        body = raw.split("#", 1)[0].split()
        if not body:
            if raw.startswith("#") and not rows and version == 0:
                header.append(raw)
            continue
        if body[0] == "version":
            version = int(body[1])
            continue
        arch, n, k, s, sm = body[0], int(body[1]), int(body[2]), int(body[3]), int(body[4])
        rows[(arch, n, k)] = (s, sm)
    return version, header, rows


def write_table(path: str, version: int, header, rows):
    lines = list(header) + ["version %d" % version]
    for (arch, n, k) in sorted(rows):
        s, sm = rows[(arch, n, k)]
        if not (1 <= s <= MAX_SPLITS and k % (64 * s) == 0 and n % 16 == 0 and 0 <= sm <= 4096):
            raise ValueError("illegal pin for %s N=%d K=%d: S=%d stream_max_m=%d" % (arch, n, k, s, sm))
        lines.append("%s %d %d %d %d" % (arch, n, k, s, sm))
    tmp = path + ".tmp%d" % os.getpid()
    with open(tmp, "w") as f:
        f.write("\n".join(lines) + "\n")
    os.replace(tmp, path)


def update_table(path: str, arch: str, n: int, k: int, pin):
    version, header, rows = read_table(path)
    rows[(arch, n, k)] = (int(pin[0]), int(pin[1]))
    write_table(path, version + 1, header, rows)


# --- measurement on the device ------------------------------------------------

def device_measure(n: int, k: int, profile, reps: int = 20, rotate_bytes: float = 2 ** 30):
    """A `measure` function timing bi_gemm_run with HIP events on cuda:0.

    Weights rotate over copies totalling `rotate_bytes` so that the Infinity
    Cache does not serve them to small-M calls.
    """
    import torch

    from . import _lib

    _lib.load()
    w0 = (torch.randn(n, k, device="cuda:0") * 0.02).to(torch.bfloat16)
    copies = max(1, int(rotate_bytes // (2 * n * k)) + 1)
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    mmax = max(m for m, _ in profile)
    x = torch.randn(mmax, k, device="cuda:0").to(torch.bfloat16)
    ys = {m: torch.empty(m, n, device="cuda:0") for m, _ in profile}

    def measure(cand):
        s, sm = cand
        hs = [_lib.Gemm(w, pin={"splits": s, "stream_max_m": sm}) for w in ws]
        out = {}
        for m, _ in profile:
            for i in range(3):
                hs[i % copies](x[:m], out=ys[m])
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                hs[i % copies](x[:m], out=ys[m])
            e1.record()
            torch.cuda.synchronize()
            out[m] = e0.elapsed_time(e1) * 1e-3 / reps
        for h in hs:
            h.close()
        return out

    return measure


def main(argv=None):
    ap = argparse.ArgumentParser(description="choose a layer's pin from its shape and a workload profile")
    ap.add_argument("--shape", required=True, help="NxK, e.g. 4096x14336")
    ap.add_argument("--profile", required=True, help="M:count,M:count,...")
    ap.add_argument("--arch", default="gfx950")
    ap.add_argument("--table", default=os.path.join(os.path.dirname(os.path.abspath(__file__)), "pins", "gfx950.txt"))
    ap.add_argument("--write", action="store_true", help="write the chosen pin into the table")
    ap.add_argument("--splits", default=",".join(map(str, SPLIT_CHOICES)))
    ap.add_argument("--stream", default=",".join(map(str, STREAM_CHOICES)))
    ap.add_argument("--reps", type=int, default=20)
    args = ap.parse_args(argv)
    n, k = (int(v) for v in args.shape.lower().split("x"))
    profile = parse_profile(args.profile)
    cands = candidates(n, k, profile, tuple(int(v) for v in args.splits.split(",")),
                       tuple(int(v) for v in args.stream.split(",")))
    measure = device_measure(n, k, profile, reps=args.reps)
    best, report = choose(profile, measure, cands)
    for (s, sm), total, t in report:
        print("S=%-2d stream_max_m=%-4d cost %.1f us  %s" % (
            s, sm, total * 1e6, " ".join("%d:%.1f" % (m, v * 1e6) for m, v in sorted(t.items()))), flush=True)
    print("chosen: N=%d K=%d splits=%d stream_max_m=%d" % (n, k, best[0], best[1]), flush=True)
    if args.write:
        update_table(args.table, args.arch, n, k, best)
        print("wrote", args.table)
    return 0


if __name__ == "__main__":
    sys.exit(main())
