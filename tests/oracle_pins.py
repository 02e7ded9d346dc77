"""The pin battery for the CPU oracle, shared by the oracle tests and the
planted-mistake tests (which run it against deliberately broken copies of the
oracle and expect it to fail).

Every check compares the oracle with something other than itself: exact
rationals, integer closed forms, numpy's fp64 matmul, hand-worked fixtures,
identity and one-hot special cases.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

import oracle
from oracle import exact
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
EPS64 = 2.0 ** -53


def wide_bf16(seed, shape, emin=-30, emax=30):
    """bf16 values spread over many binades, random signs (no subnormals)."""
    g = synth.rng(seed)
    mant = g.uniform(1.0, 2.0, size=shape).astype(np.float32)
    e = g.integers(emin, emax + 1, size=shape)
    s = np.where(g.random(size=shape) < 0.5, -1.0, 1.0)
    v = (s * mant * np.exp2(e)).astype(np.float32)
    zero = g.random(size=shape) < 0.1
    v[zero] = 0.0
    return synth.f32_to_bf16_bits(v)


def load_gemm_golden():
    cases, cur, sect = [], None, None
    for line in open(os.path.join(GOLDEN, "tiny_gemm.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("case "):
            cur = {"name": line[5:], "x": [], "w": [], "y": [], "a": []}
            cases.append(cur)
            continue
        if line in ("x", "w", "y", "a"):
            sect = line
            continue
        cur[sect].append([float(t) for t in line.split()])
    return cases


def load_fold_golden():
    out = []
    for line in open(os.path.join(GOLDEN, "fold_fp32.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        lhs, rhs = line.split("->")
        parts = np.array([int(t, 16) for t in lhs.split()], dtype=np.uint32).view(np.float32)
        out.append((parts, int(rhs.strip(), 16)))
    return out


# --- individual pins; each returns None or raises AssertionError -------------

def pin_exact_rationals(lib=None):
    for seed, (m, n, k) in enumerate([(1, 1, 1), (2, 3, 7), (4, 4, 64), (3, 2, 33), (4, 1, 48)]):
        x = wide_bf16(100 + seed, (m, k))
        w = wide_bf16(200 + seed, (n, k))
        y, a = oracle.gemm_f64(x, w, lib=lib)
        ye, ae = exact.gemm_exact(x, w)
        for i in range(m):
            for j in range(n):
                bound = Fraction(max(k - 1, 0)) * Fraction(EPS64) * ae[i][j]
                assert abs(Fraction(y[i, j]) - ye[i][j]) <= bound, (seed, i, j)
                assert abs(Fraction(a[i, j]) - ae[i][j]) <= bound, (seed, i, j)


def pin_golden_gemm(lib=None):
    for c in load_gemm_golden():
        x = synth.f32_to_bf16_bits(np.array(c["x"], np.float32))
        w = synth.f32_to_bf16_bits(np.array(c["w"], np.float32))
        assert np.array_equal(synth.bf16_bits_to_f32(x), np.array(c["x"], np.float32)), "fixture not exact in bf16"
        y, a = oracle.gemm_f64(x, w, lib=lib)
        assert np.array_equal(y, np.array(c["y"])), c["name"]
        assert np.array_equal(a, np.array(c["a"])), c["name"]


def pin_integer_closed_forms(lib=None):
    # all ones: every entry is K
    for k in (1, 7, 512, 14336):
        x = synth.f32_to_bf16_bits(np.ones((2, k), np.float32))
        w = synth.f32_to_bf16_bits(np.ones((3, k), np.float32))
        y, a = oracle.gemm_f64(x, w, lib=lib)
        assert np.all(y == k) and np.all(a == k)
        assert np.all(oracle.gemm_i64(x, w, lib=lib) == k)
    # x = 1, w[n][k] = (k mod 7) - 3: whole periods sum to 0, the rest r terms
    # sum to r(r-1)/2 - 3r
    for k in (5, 14, 100, 3584):
        r = k % 7
        expect = r * (r - 1) // 2 - 3 * r
        x = synth.f32_to_bf16_bits(np.ones((1, k), np.float32))
        wv = (np.arange(k) % 7 - 3).astype(np.float32)
        w = synth.f32_to_bf16_bits(np.stack([wv, -wv]))
        y, _ = oracle.gemm_f64(x, w, lib=lib)
        assert y[0, 0] == expect and y[0, 1] == -expect, (k, y, expect)
        yi = oracle.gemm_i64(x, w, lib=lib)
        assert yi[0, 0] == expect and yi[0, 1] == -expect
    # x[i][k] = i+1 (rows scale), w[n][k] = 1 if k <= n else 0: y = (i+1)(n+1)
    m, n, k = 3, 5, 8
    x = synth.f32_to_bf16_bits(np.repeat(np.arange(1, m + 1, dtype=np.float32)[:, None], k, 1))
    w = synth.f32_to_bf16_bits(np.tril(np.ones((n, k), np.float32)))
    y, _ = oracle.gemm_f64(x, w, lib=lib)
    assert np.array_equal(y, np.outer(np.arange(1, m + 1), np.arange(1, n + 1)).astype(float))


def pin_integer_random(lib=None):
    for seed, (m, n, k) in enumerate([(5, 7, 512), (3, 16, 14336), (2, 9, 3584)]):
        x = synth.int_bf16(300 + seed, (m, k))
        w = synth.int_bf16(400 + seed, (n, k))
        xi = synth.bf16_bits_to_f32(x).astype(np.int64)
        wi = synth.bf16_bits_to_f32(w).astype(np.int64)
        ref = xi @ wi.T  # numpy int64 matmul: an independent routine
        assert np.array_equal(oracle.gemm_i64(x, w, lib=lib), ref)
        y, a = oracle.gemm_f64(x, w, lib=lib)
        assert np.array_equal(y, ref.astype(np.float64))
        assert np.array_equal(a, (np.abs(xi) @ np.abs(wi).T).astype(np.float64))


def pin_numpy_fp64(lib=None):
    for seed, (m, n, k) in enumerate([(8, 16, 512), (3, 40, 4096), (2, 6, 14336)]):
        x = synth.normal_bf16(500 + seed, (m, k))
        w = synth.normal_bf16(600 + seed, (n, k), 0.02)
        xf = synth.bf16_bits_to_f32(x).astype(np.float64)
        wf = synth.bf16_bits_to_f32(w).astype(np.float64)
        y, a = oracle.gemm_f64(x, w, lib=lib)
        ref = xf @ wf.T
        aref = np.abs(xf) @ np.abs(wf).T
        bound = 2 * k * EPS64 * aref
        assert np.all(np.abs(y - ref) <= bound)
        assert np.all(np.abs(a - aref) <= bound)


def pin_identity_onehot(lib=None):
    k = 96
    x = synth.normal_bf16(700, (5, k))
    eye = synth.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
    y, _ = oracle.gemm_f64(x, eye, lib=lib)
    assert np.array_equal(y, synth.bf16_bits_to_f32(x).astype(np.float64))
    w = synth.normal_bf16(701, (11, k), 0.02)
    onehot = synth.f32_to_bf16_bits(np.eye(k, dtype=np.float32)[[0, 17, 95]])
    y, _ = oracle.gemm_f64(onehot, w, lib=lib)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    assert np.array_equal(y, wf[:, [0, 17, 95]].T)


def pin_row_selection(lib=None):
    x = synth.normal_bf16(800, (37, 64))
    w = synth.normal_bf16(801, (9, 64), 0.02)
    rows = np.array([36, 0, 5, 5, 17])
    y, a = oracle.gemm_f64(x, w, rows=rows, lib=lib)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)[rows]
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    assert np.all(np.abs(y - xf @ wf.T) <= 2 * 64 * EPS64 * (np.abs(xf) @ np.abs(wf).T))


def pin_grouped(lib=None):
    # tiny exact case with empty experts and uneven groups
    e, n, k = 4, 3, 16
    offsets = np.array([0, 2, 2, 5, 6], np.int32)
    x = wide_bf16(900, (6, k), -10, 10)
    w = wide_bf16(901, (e, n, k), -10, 10)
    y, a = oracle.grouped_f64(x, w, offsets, lib=lib)
    owner = [0, 0, 2, 2, 2, 3]
    for r in range(6):
        ye, ae = exact.gemm_exact(x[r:r + 1], w[owner[r]])
        for j in range(n):
            bound = Fraction(k - 1) * Fraction(EPS64) * ae[0][j]
            assert abs(Fraction(y[r, j]) - ye[0][j]) <= bound, (r, j)
            assert abs(Fraction(a[r, j]) - ae[0][j]) <= bound, (r, j)
    # larger: against numpy per expert, from a real routing table
    tok, off, _ = synth.moe_routing(902, 16, experts=8, topk=2)
    k = 128
    xt = synth.normal_bf16(903, (16, k))
    x = xt[tok]
    w = synth.normal_bf16(904, (8, 5, k), 0.02)
    y, _ = oracle.grouped_f64(x, w, off, lib=lib)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    for ex in range(8):
        lo, hi = off[ex], off[ex + 1]
        ref = xf[lo:hi] @ wf[ex].T
        bound = 2 * k * EPS64 * (np.abs(xf[lo:hi]) @ np.abs(wf[ex]).T)
        assert np.all(np.abs(y[lo:hi] - ref) <= bound), ex


def pin_fold(lib=None):
    for parts, want in load_fold_golden():
        got = oracle.fold_f32(parts.reshape(-1, 1), lib=lib)
        assert int(got.view(np.uint32)[0]) == want, (parts, hex(int(got.view(np.uint32)[0])), hex(want))


def pin_moe_topk(lib=None):
    """Routing against a plain sort, closed-form weights and shift invariance."""
    for seed, t, e, k, step in ((910, 40, 16, 4, 0.5), (911, 20, 9, 9, 0.25), (912, 30, 128, 8, 0.0)):
        lg = synth.router_logits(seed, t, e, step=step)
        ids, w = oracle.moe_topk(lg, k, lib=lib)
        for i in range(t):
            want = sorted(range(e), key=lambda q: (-float(lg[i, q]), q))[:k]
            assert ids[i].tolist() == want, (seed, i)
        assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
        assert np.all(np.diff(w, axis=1) <= 0)
        # adding a constant that keeps every logit exact changes nothing
        if step > 0:
            ids2, w2 = oracle.moe_topk(lg + np.float32(0.5), k, lib=lib)
            assert np.array_equal(ids, ids2) and np.allclose(w, w2, rtol=0, atol=1e-15)
    # all logits equal: the k lowest ids, weight 1/k each
    ids, w = oracle.moe_topk(np.full((2, 10), 0.75, np.float32), 4, lib=lib)
    assert ids.tolist() == [[0, 1, 2, 3]] * 2 and np.all(w == 0.25)
    # two chosen logits ln(3) apart: weights 3/4 and 1/4 (up to the fp32 logit)
    l3 = np.float32(np.log(3.0))
    ids, w = oracle.moe_topk(np.array([[0.0, l3, -5.0]], np.float32), 2, lib=lib)
    assert ids.tolist() == [[1, 0]] and abs(w[0, 0] - 0.75) < 1e-7 and abs(w[0, 1] - 0.25) < 1e-7
    try:
        oracle.moe_topk(np.array([[0.0, np.inf]], np.float32), 1, lib=lib)
    except ValueError:
        pass
    else:
        raise AssertionError("a non-finite logit must be rejected")


def pin_moe_permute(lib=None):
    """Grouping against numpy's stable sort by expert, and its inverse."""
    for seed, t, e, k in ((920, 50, 16, 4), (921, 7, 128, 8), (922, 1, 8, 8)):
        g = synth.rng(seed)
        ids = np.stack([g.permutation(e)[:k] for _ in range(t)]).astype(np.int32)
        off, tok, row_of = oracle.moe_permute(ids, e, lib=lib)
        flat = ids.reshape(-1)
        order = np.argsort(flat, kind="stable")
        assert np.array_equal(tok, (order // k).astype(np.int32))
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=e))]))
        inv = np.empty(t * k, np.int64)
        inv[order] = np.arange(t * k)
        assert np.array_equal(row_of.reshape(-1), inv)
        assert np.array_equal(tok[row_of], np.repeat(np.arange(t), k).reshape(t, k))
    try:
        oracle.moe_permute(np.array([[0, 9]], np.int32), 8, lib=lib)
    except ValueError:
        pass
    else:
        raise AssertionError("an id outside 0..E-1 must be rejected")


def pin_swiglu(lib=None):
    """Closed forms of silu(g) * u and scipy's logistic function."""
    from scipy.special import expit

    l3 = float(np.float32(np.log(3.0)))
    gates = [0.0, l3, 30.0, -30.0, 1.0]
    ups = [3.0, 0.5, 2.0, 2.0, 0.0]
    a = oracle.swiglu_f64(np.array([gates + ups], np.float32), lib=lib)[0]
    assert a[0] == 0.0                                      # silu(0) = 0
    assert abs(a[1] / (0.375 * l3) - 1.0) < 1e-7            # silu(ln 3) = 3/4 ln 3, times 1/2
    assert abs(a[2] / 60.0 - 1.0) < 1e-12                   # large gate: g * u
    assert -1e-11 < a[3] < 0.0                              # very negative gate: ~0, negative
    assert a[4] == 0.0                                      # up 0 -> 0
    g = synth.rng(930).standard_normal((40, 64)).astype(np.float32) * 4
    a = oracle.swiglu_f64(g, lib=lib)
    gg, uu = g[:, :32].astype(np.float64), g[:, 32:].astype(np.float64)
    assert np.allclose(a, gg * expit(gg) * uu, rtol=1e-14, atol=1e-300)


def pin_moe_combine(lib=None):
    """Integer outputs with dyadic weights sum exactly in any order."""
    g = synth.rng(940)
    t, k, h, r = 12, 4, 24, 48
    o = g.integers(-3, 4, size=(r, h)).astype(np.float32)
    w = np.exp2(-g.integers(0, 4, size=(t, k))).astype(np.float32)
    row_of = np.stack([g.permutation(r)[:k] for _ in range(t)]).astype(np.int32)
    y, s = oracle.moe_combine_f64(o, w, row_of, lib=lib)
    for i in range(t):
        for n in range(h):
            want = sum(Fraction(float(w[i, j])) * Fraction(float(o[row_of[i, j], n])) for j in range(k))
            assert Fraction(y[i, n]) == want
            assert s[i, n] == float(sum(abs(Fraction(float(w[i, j])) * Fraction(float(o[row_of[i, j], n])))
                                        for j in range(k)))
    # one expert with weight 1 returns its row
    y1, _ = oracle.moe_combine_f64(o, np.ones((t, 1), np.float32), row_of[:, :1], lib=lib)
    assert np.array_equal(y1, o[row_of[:, 0]].astype(np.float64))


def pin_rmsnorm(lib=None):
    """RMSNorm against closed forms, scale invariance, exact rational sums of
    squares and numpy's fp64 formula."""
    h = 64
    one = synth.f32_to_bf16_bits(np.ones(h, np.float32))
    # a constant row c: ms = c^2, y = g * c / sqrt(c^2 + eps); with eps = 0 it is g * sign(c)
    for c in (3.0, -0.5, 2.0 ** -20):
        x = synth.f32_to_bf16_bits(np.full((1, h), c, np.float32))
        y, ms = oracle.rmsnorm_f64(x, one, 0.0, lib=lib)
        assert ms[0] == c * c and np.all(y == np.sign(c)), (c, y[0, :3])
        y, _ = oracle.rmsnorm_f64(x, one, 1e-5, lib=lib)
        assert np.allclose(y, c / np.sqrt(c * c + 1e-5), rtol=1e-15, atol=0)
    # one nonzero entry v at k: ms = v^2 / H, y[k] = g[k] * sqrt(H) * sign(v), others 0
    g = synth.normal_bf16(950, (h,), 1.0)
    gf = synth.bf16_bits_to_f32(g).astype(np.float64)
    x = np.zeros((1, h), np.uint16)
    x[0, 5] = synth.f32_to_bf16_bits(np.array([-0.75], np.float32))[0]
    y, ms = oracle.rmsnorm_f64(x, g, 0.0, lib=lib)
    assert ms[0] == 0.5625 / h
    assert abs(y[0, 5] / (-gf[5] * np.sqrt(h)) - 1) < 1e-15 and np.all(np.delete(y[0], 5) == 0)
    # scaling a row by a power of two changes nothing when eps = 0
    x = synth.normal_bf16(951, (4, h))
    xs = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x) * np.float32(8.0))
    y1, _ = oracle.rmsnorm_f64(x, g, 0.0, lib=lib)
    y2, _ = oracle.rmsnorm_f64(xs, g, 0.0, lib=lib)
    assert np.array_equal(y1, y2)
    # the mean of squares against exact rationals
    x = synth.normal_bf16(952, (3, 40))
    _, ms = oracle.rmsnorm_f64(x, synth.f32_to_bf16_bits(np.ones(40, np.float32)), 0.0, lib=lib)
    for t in range(3):
        exact = sum(Fraction(float(v)) ** 2 for v in synth.bf16_bits_to_f32(x[t])) / 40
        assert abs(Fraction(ms[t]) - exact) <= exact * Fraction(1, 2 ** 50)
    # numpy's fp64 formula, an independent library routine
    x = synth.normal_bf16(953, (7, 96), 3.0)
    g = synth.normal_bf16(954, (96,), 0.3)
    y, _ = oracle.rmsnorm_f64(x, g, 1e-6, lib=lib)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    want = xf * synth.bf16_bits_to_f32(g).astype(np.float64) / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + 1e-6)
    assert np.allclose(y, want, rtol=1e-14, atol=0)


def pin_decode_attn(lib=None):
    """Decode attention against closed forms (one key; equal keys or q = 0
    give the mean of the values; one dominant key), the grouped-head mapping,
    scipy's softmax and key-order invariance."""
    from scipy.special import softmax

    f = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64)  # noqa: E731
    b16 = lambda a: synth.f32_to_bf16_bits(np.asarray(a, np.float32))  # noqa: E731
    d = 16
    # one key: the output is its value; an empty sequence gives zeros
    q = synth.normal_bf16(960, (2, 4, d))
    k = synth.normal_bf16(961, (1, 2, d))
    v = synth.normal_bf16(962, (1, 2, d))
    o, mg, _ = oracle.decode_attn_f64(q, k, v, np.array([0, 1, 1], np.int32), 0.25, lib=lib)
    for h in range(4):
        assert np.array_equal(o[0, h], f(v[0, h // 2])) and np.array_equal(mg[0, h], np.abs(f(v[0, h // 2])))
    assert np.all(o[1] == 0)
    # equal keys, or q = 0: every weight 1/n, the output is the mean of the values
    n = 8
    v = synth.normal_bf16(963, (n, 1, d))
    keq = np.repeat(synth.normal_bf16(964, (1, 1, d)), n, axis=0)
    qz = np.zeros((1, 2, d), np.uint16)
    want = np.array([float(sum(Fraction(float(x)) for x in f(v[:, 0, i])) / n) for i in range(d)])
    for qq, kk in ((synth.normal_bf16(965, (1, 2, d)), keq), (qz, synth.normal_bf16(966, (n, 1, d)))):
        o, _, _ = oracle.decode_attn_f64(qq, kk, v, np.array([0, n], np.int32), 0.5, lib=lib)
        assert np.allclose(o[0, 0], want, rtol=0, atol=1e-15) and np.allclose(o[0, 1], want, rtol=0, atol=1e-15)
    # one dominant key: its score exceeds the others' by 200, so the output is its value
    k = np.zeros((n, 1, d), np.uint16)
    k[3, 0, 0] = b16([200.0])[0]
    q = np.zeros((1, 1, d), np.uint16)
    q[0, 0, 0] = b16([1.0])[0]
    o, _, qk = oracle.decode_attn_f64(q, k, v, np.array([0, n], np.int32), 1.0, lib=lib)
    assert np.allclose(o[0, 0], f(v[3, 0]), rtol=1e-12, atol=1e-80) and qk[0, 0] == 200.0
    # grouped heads: query head h reads kv head h // (Hq / Hkv); values constant per kv head
    hq, hkv, n = 8, 4, 5
    v = np.stack([b16(np.full((hkv, d), 0.0) + np.arange(hkv)[:, None] + 1) for _ in range(n)])
    k = synth.normal_bf16(967, (n, hkv, d))
    q = synth.normal_bf16(968, (1, hq, d))
    o, _, _ = oracle.decode_attn_f64(q, k, v, np.array([0, n], np.int32), 0.25, lib=lib)
    for h in range(hq):
        assert np.allclose(o[0, h], h // 2 + 1, rtol=1e-15, atol=0), h
    # scipy's softmax, ragged sequences; and key order does not matter
    hq, hkv, d = 6, 2, 32
    st = np.array([0, 7, 7, 20, 21], np.int32)
    q = synth.normal_bf16(969, (4, hq, d))
    k = synth.normal_bf16(970, (21, hkv, d), 2.0)
    v = synth.normal_bf16(971, (21, hkv, d))
    sc = 1.0 / np.sqrt(d)
    o, _, _ = oracle.decode_attn_f64(q, k, v, st, sc, lib=lib)
    for b in range(4):
        for h in range(hq):
            ks, vs = f(k[st[b]:st[b + 1], h // 3]), f(v[st[b]:st[b + 1], h // 3])
            if len(ks) == 0:
                assert np.all(o[b, h] == 0)
                continue
            assert np.allclose(o[b, h], softmax(sc * (ks @ f(q[b, h]))) @ vs, rtol=1e-13, atol=1e-15)
    perm = np.concatenate([np.arange(7), 7 + synth.rng(972).permutation(13), [20]])
    o2, _, _ = oracle.decode_attn_f64(q, k[perm], v[perm], st, sc, lib=lib)
    assert np.allclose(o, o2, rtol=1e-13, atol=1e-15)


ALL_PINS = [
    pin_exact_rationals,
    pin_golden_gemm,
    pin_integer_closed_forms,
    pin_integer_random,
    pin_numpy_fp64,
    pin_identity_onehot,
    pin_row_selection,
    pin_grouped,
    pin_fold,
    pin_moe_topk,
    pin_moe_permute,
    pin_swiglu,
    pin_moe_combine,
    pin_rmsnorm,
    pin_decode_attn,
]
