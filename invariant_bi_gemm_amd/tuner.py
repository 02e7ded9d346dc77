"""Offline pin tuner: choose one layer's pin from its shape and a workload profile.

The pin of a layer (N, K) is its reduction tree -- the number S of contiguous
equal K splits -- plus its tiling: which dense kernel (output block shape,
streaming or tiled) serves each range of row counts M.  Both are fixed before
deployment and never read the batch (Detent, §3: pins and knobs form a
commitment tuple fixed for a workload; §6: the tuner picks it per workload).
The tiling only moves work between kernels that realise the same tree, so it
never changes an output bit; S does.

Cost model (Detent, §6 eq. 3): a workload profile W = {(M, n)} lists the row
counts its calls have and how often; the cost of a legal assignment a is
T(a) = sum over W of n * t(M, a), with t measured on the device; the tuner
returns argmin T.  An assignment is a tree S and a kernel per profile M.
Given S, the kernels of different M do not interact, so the argmin picks the
fastest kernel at each M, and the tree with the lowest resulting total.
Candidates are legal by construction (S divides K into whole 64-wide stages;
the library checks it again); each is measured by creating a handle with
the pin swapped in (Detent, §6 "Search": a repin swaps the constants
without solving again).  The grids are small, so the search is exhaustive,
except that the weight streamers are not tried above 256 rows (they re-read
W once per 16 rows per m-block there) -- a measured family of the pages is
likewise a handful of candidates (Detent, §6 Fig. 6).

Between two profile points the tiling switches at their geometric mean; the
last kernel serves every larger M.

Usage:
    python -m invariant_bi_gemm_amd.tuner --shape 4096x14336 \
        --profile 1:8,2:8,4:8,8:8,16:8,32:4,64:4,128:2,256:2,512:1,1024:1,2048:1,4096:1,8192:1 \
        --table invariant_bi_gemm_amd/pins/gfx950.txt --write

The table keeps one line per (arch, N, K); writing replaces the shape's line,
keeps the others, bumps the version (a new table version may give different
bits, as a different commitment tuple does) and names the library's tree.
"""
from __future__ import annotations

import argparse
import math
import os
import sys

SPLIT_CHOICES = (1, 2, 4, 7, 8, 14, 16)
MAX_SPLITS = 16
STREAM_KINDS = ("stream_mb1", "stream_mb2", "stream_mb4", "stream_mb2_n2", "stream_mb4_n2", "stream_mb2_n4",
                "stream_mb4_n4")
KERNEL_KINDS = ("stream_mb1", "stream_mb2", "stream_mb4", "tiled_64x32", "tiled_64x64", "tiled_128x64",
                "tiled_128x64_deep", "tiled_128x128", "tiled_128x128_deep", "tiled4_128x256", "tiled4_256x256",
                "tiled4_160x256", "tiled4_192x256", "stream_mb2_n2", "stream_mb4_n2", "stream_mb2_n4",
                "stream_mb4_n4")
STREAM_LIMIT = 256  # streamers are candidates at M <= this,
WIDE_STREAM_LIMIT = 1024  # those over 32- and 64-column strips at M <= this
WIDE_STREAM_KINDS = ("stream_mb2_n2", "stream_mb4_n2", "stream_mb2_n4", "stream_mb4_n4")
MAX_TILINGS = 12
INT32_MAX = 2 ** 31 - 1


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


CS = "+cs"        # a kind running the tree's splits concurrently (S > 1 only)
CS_LIMIT = 16384  # the library's bound on the rows of such an entry


def base_kind(kd: str) -> str:
    return kd[:-len(CS)] if kd.endswith(CS) else kd


def kernel_candidates(m: int, kinds=KERNEL_KINDS):
    """Kernel kinds tried at M rows."""
    def fits(kd):
        kd = base_kind(kd)
        if kd in WIDE_STREAM_KINDS:
            return m <= WIDE_STREAM_LIMIT
        return m <= STREAM_LIMIT or kd not in STREAM_KINDS

    return [kd for kd in kinds if fits(kd)]


def tree_kinds(s: int, kinds=KERNEL_KINDS):
    """The kinds measured for a tree with s splits: with s > 1 each kind also
    with its splits run concurrently."""
    return list(kinds) + ([kd + CS for kd in kinds] if s > 1 else [])


def cost(profile, timing):
    """Detent eq. 3: sum of count * time over the profile."""
    return sum(n * timing[m] for m, n in profile)


TIE = 0.03        # kernels within 3% of the fastest count as equally fast,
TIE_ABS = 0.5e-6  # and so do kernels within half a microsecond (launch jitter)


def pick_kernels(times, kinds=KERNEL_KINDS, tie=TIE, tie_abs=TIE_ABS):
    """{M: {kind: seconds}} -> {M: (kind, seconds)}, ascending in M: the
    fastest kind, except that the kind of the previous M is kept while it is
    within `tie` (relative) or `tie_abs` (seconds) of the fastest: timings of
    equally fast kernels differ by noise, which would otherwise cut the
    tiling into many small ranges.  Ties between new kinds go to the earlier
    kind."""
    out, prev = {}, None
    for m in sorted(times):
        cand = [(t, kinds.index(kd), kd) for kd, t in times[m].items() if kd in kinds and kd in kernel_candidates(m, kinds)]
        best_t = min(c[0] for c in cand)
        if prev is not None and prev in times[m] and prev in kernel_candidates(m, kinds) and \
                times[m][prev] <= max(best_t * (1 + tie), best_t + tie_abs):
            out[m] = (prev, times[m][prev])
        else:
            t, _, kd = min(cand)
            out[m] = (kd, t)
        prev = out[m][0]
    return out


def choose(profile, measure, splits, kinds=KERNEL_KINDS, tie=TIE):
    """argmin over trees S and per-M kernels of the profile cost.

    ``measure(s, kind)`` returns {M: seconds} for the profile's M (only the
    M where ``kind`` is a candidate are read).  Returns (S, {M: kind},
    {M: seconds}, report) with report = [(S, total, {M: (kind, seconds)},
    {M: {kind: seconds}})], the last the times of every candidate measured.
    Per S the kernels are those of pick_kernels; ties between trees go to
    the earlier candidate (fewer splits)."""
    report = []
    best = None
    mmax = max(m for m, _ in profile)
    for s in splits:
        skinds = tree_kinds(s, kinds)
        times = {m: {} for m, _ in profile}
        for kd in skinds:
            t = measure(s, kd)
            for m, _ in profile:
                # the last range covers every larger M: no concurrent splits there
                if kd in kernel_candidates(m, skinds) and not (kd.endswith(CS) and (m == mmax or m > CS_LIMIT)):
                    times[m][kd] = t[m]
        kinds_ = skinds
        per_m = pick_kernels(times, kinds_, tie)
        # a tiling list holds at most MAX_TILINGS ranges: widen the tie until
        # the picks fit (only noise-level differences are ever merged first)
        t_ = tie
        while len(tiling_from_choice({m: v[0] for m, v in per_m.items()}, check=False)) > MAX_TILINGS:
            t_ *= 2
            per_m = pick_kernels(times, kinds_, t_)
        total = cost(profile, {m: v[1] for m, v in per_m.items()})
        report.append((s, total, per_m, times))
        if best is None or total < best[1]:
            best = (s, total, per_m)
    s, _, per_m = best
    return s, {m: v[0] for m, v in per_m.items()}, {m: v[1] for m, v in per_m.items()}, report


def tiling_from_choice(choice, check=True):
    """{M: kind} at the profile points -> [(m_max, kind)], the switch between
    neighbouring points at their geometric mean, equal neighbours merged, the
    last bound None (every larger M)."""
    ms = sorted(choice)
    out = []
    for i, m in enumerate(ms):
        bound = None if i + 1 == len(ms) else int(math.floor(math.sqrt(m * ms[i + 1])))
        if out and out[-1][1] == choice[m]:
            out[-1] = (bound, choice[m])
        else:
            out.append((bound, choice[m]))
    if check and len(out) > MAX_TILINGS:
        raise ValueError("the tiling needs %d entries, at most %d fit" % (len(out), MAX_TILINGS))
    return out


def stream_threshold(tiling, default=16):
    """The largest M the tiling streams (grouped handles stream experts up to
    it); `default` when it streams nothing."""
    last = 0
    for bound, kind in tiling:
        if base_kind(kind) in STREAM_KINDS:
            last = bound if bound is not None else 4096
    return min(last, 4096) if last else default


def format_tiling(tiling):
    return ",".join("%s:%s" % ("*" if b is None else b, kd) for b, kd in tiling)


def parse_tiling(text: str):
    out = []
    for item in text.split(","):
        b, _, kd = item.partition(":")
        if base_kind(kd) not in KERNEL_KINDS:
            raise ValueError("unknown kernel kind %r" % kd)
        out.append((None if b == "*" else int(b), kd))
    bounds = [b for b, _ in out[:-1]]
    if not out or out[-1][0] is not None or bounds != sorted(set(bounds)) or any(b < 1 for b in bounds):
        raise ValueError("tiling bounds must ascend and end with '*': %r" % text)
    if out[-1][1].endswith(CS) or any(kd.endswith(CS) and b > CS_LIMIT for b, kd in out[:-1]):
        raise ValueError("concurrent splits only on bounded entries of at most %d rows: %r" % (CS_LIMIT, text))
    return out


# --- pin table ---------------------------------------------------------------

def read_table(path: str):
    """-> (version, tree, header comment lines, {(arch, N, K): (splits, stream_max_m, tiling)})."""
    version = 0
    tree = None
    header = []
    rows = {}
    if not os.path.exists(path):
        return version, tree, header, rows
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
        if body[0] == "tree":
            tree = body[1]
            continue
        arch, n, k, s, sm = body[0], int(body[1]), int(body[2]), int(body[3]), int(body[4])
        tiling = parse_tiling(body[5]) if len(body) > 5 else []
        rows[(arch, n, k)] = (s, sm, tiling)
    return version, tree, header, rows


def write_table(path: str, version: int, tree: str, header, rows):
    lines = list(header) + ["version %d" % version, "tree %s" % tree]
    for (arch, n, k) in sorted(rows):
        s, sm, tiling = rows[(arch, n, k)]
        if not (1 <= s <= MAX_SPLITS and k % (64 * s) == 0 and n % 16 == 0 and 0 <= sm <= 4096):
            raise ValueError("illegal pin for %s N=%d K=%d: S=%d stream_max_m=%d" % (arch, n, k, s, sm))
        line = "%s %d %d %d %d" % (arch, n, k, s, sm)
        if tiling:
            parse_tiling(format_tiling(tiling))  # validates
            line += " " + format_tiling(tiling)
        lines.append(line)
    tmp = path + ".tmp%d" % os.getpid()
    with open(tmp, "w") as f:
        f.write("\n".join(lines) + "\n")
    os.replace(tmp, path)


def update_table(path: str, arch: str, n: int, k: int, pin, tree: str):
    """pin = (splits, stream_max_m, tiling)."""
    version, _, header, rows = read_table(path)
    rows[(arch, n, k)] = (int(pin[0]), int(pin[1]), list(pin[2]))
    write_table(path, version + 1, tree, header, rows)


# --- measurement on the device ------------------------------------------------

def device_measure(n: int, k: int, profile, reps: int = 20, rotate_bytes: float = 2 ** 30, batches: int = 3):
    """A `measure(s, kind)` function timing bi_gemm_run with HIP events on
    cuda:0, the kernel forced by a one-entry tiling list: per M, the fastest
    of `batches` batches of `reps` back-to-back calls (the mean of a batch),
    the calls made straight through the C ABI with prepared arguments so the
    host keeps ahead of the GPU.

    Weights rotate over copies totalling `rotate_bytes` so that the Infinity
    Cache does not serve them to small-M calls.
    """
    import ctypes

    import torch

    from . import _lib

    lib = _lib.load()
    w0 = (torch.randn(n, k, device="cuda:0") * 0.02).to(torch.bfloat16)
    copies = max(1, int(rotate_bytes // (2 * n * k)) + 1)
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    mmax = max(m for m, _ in profile)
    x = torch.randn(mmax, k, device="cuda:0").to(torch.bfloat16)
    ys = {m: torch.empty(m, n, device="cuda:0") for m, _ in profile}
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    xp = ctypes.c_void_p(x.data_ptr())
    run = lib.bi_gemm_run

    cs_rows = min(mmax, CS_LIMIT)

    def measure(s, kind):
        # a kind with concurrent splits serves every measured M up to the
        # largest (its workspace sized for it); the plain kind covers the rest
        tiling = [(cs_rows, kind), (None, base_kind(kind))] if kind.endswith(CS) else [(None, kind)]
        hs = [_lib.Gemm(w, pin={"splits": s, "stream_max_m": 0, "tiling": tiling}) for w in ws]
        hp = [h._h for h in hs]
        out = {}
        for m, _ in profile:
            if kind not in kernel_candidates(m, [kind]):
                out[m] = float("inf")
                continue
            yp = ctypes.c_void_p(ys[m].data_ptr())
            for i in range(3):
                _lib.check(run(hp[i % copies], xp, m, yp, stream))
            torch.cuda.synchronize()
            best = float("inf")
            for _ in range(batches):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(reps):
                    run(hp[i % copies], xp, m, yp, stream)
                e1.record()
                torch.cuda.synchronize()
                best = min(best, e0.elapsed_time(e1) * 1e-3 / reps)
            out[m] = best
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
    ap.add_argument("--kinds", default=",".join(KERNEL_KINDS))
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--show", type=int, default=5, help="candidates listed per M in the report (fastest first)")
    args = ap.parse_args(argv)
    n, k = (int(v) for v in args.shape.lower().split("x"))
    profile = parse_profile(args.profile)
    kinds = tuple(v for v in args.kinds.split(",") if v)
    for kd in kinds:
        if kd not in KERNEL_KINDS:
            raise SystemExit("unknown kernel kind %r (concurrent variants are added for S > 1)" % kd)
    splits = legal_splits(k, tuple(int(v) for v in args.splits.split(",")))
    measure = device_measure(n, k, profile, reps=args.reps)
    s, choice, times, report = choose(profile, measure, splits, kinds)
    for s_, total, per_m, cand in report:
        print("S=%-2d cost %.1f us  %s" % (s_, total * 1e6, " ".join(
            "%d:%s:%.1f" % (m, kd, t * 1e6) for m, (kd, t) in sorted(per_m.items()))), flush=True)
        for m in sorted(cand):
            fastest = sorted(cand[m].items(), key=lambda kv: kv[1])[:args.show]
            print("    M=%-6d %s" % (m, "  ".join("%s %.1f" % (kd, t * 1e6) for kd, t in fastest)), flush=True)
    tiling = tiling_from_choice(choice)
    smax = stream_threshold(tiling)
    print("chosen: N=%d K=%d splits=%d stream_max_m=%d tiling=%s" % (n, k, s, smax, format_tiling(tiling)),
          flush=True)
    if args.write:
        from . import _lib

        tree = _lib.load().bi_gemm_tree_id().decode()
        update_table(args.table, args.arch, n, k, (s, smax, tiling), tree)
        print("wrote", args.table)
    return 0


if __name__ == "__main__":
    sys.exit(main())
