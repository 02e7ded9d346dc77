"""The MoE expert layer around the grouped GEMM on the GPU (gpu).

Each step is compared with the oracle on seeded inputs: top-k routing (ids
exact, weights within a derived fp32 bound), grouping by expert (exact), row
gather (exact), SwiGLU (the bf16 rounding of the fp64 value, or its neighbour
where the fp32 evaluation may straddle a rounding midpoint) and the weighted
combine (within the fp32 bound of a k-term sum, and bit for bit the fp32 sum
in ascending expert id that the header specifies).  The whole layer is
checked three ways: against a chain of oracle steps within a bound derived
step by step; bit for bit against the same steps called one by one through
the C ABI; and for batch invariance: a token's output bits do not change
with the token count, its position or the other tokens.

Shapes are those of a Qwen3-30B-A3B-style layer (128 experts, top-8, hidden
2048, expert width 768), the workload the grouped GEMM is measured on.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, assert_bits_equal, bits32, to_dev

pytestmark = pytest.mark.gpu

E, TOPK, H, I = 128, 8, 2048, 768
U24 = 2.0 ** -24


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def bf16_host(t):
    """bf16 device tensor -> its uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_value(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def round_bf16(x, mode=np.rint):
    """fp64 -> the nearest bf16 value (8 significant bits), exactly, with
    ``mode`` np.rint (ties to even), np.floor or np.ceil on the significand."""
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(mode(np.ldexp(m, 8)), e - 8)


# --------------------------------------------------------------------------
# top-k routing
# --------------------------------------------------------------------------

def topk_weight_bound(lg, ids, k):
    """Relative error bound of the fp32 weights exp(l_j - l_0) / sum exp(...):
    the subtraction, exp and k-term sum each add a few ulps; the exponent's
    rounding error grows with |l_j - l_0|."""
    chosen = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), axis=1)
    d = np.abs(chosen - chosen[:, :1]).max(axis=1, keepdims=True)
    return (k + 8 + d) * 2 * U24


@pytest.mark.parametrize("experts,k,tokens,step", [
    (128, 8, 1, 0.0),
    (128, 8, 300, 0.0),
    (128, 8, 300, 0.25),    # many equal logits: the tie rule decides
    (64, 1, 77, 0.0),
    (16, 16, 33, 0.5),      # k == E: every expert, in rank order
    (1024, 64, 9, 0.125),   # the largest E and k
    (200, 5, 5, 0.0),       # E not a multiple of 64
])
def test_topk_matches_oracle(gpu, experts, k, tokens, step):
    lg = synth.router_logits(300 + experts + k, tokens, experts, step)
    ids, w = gpu.moe_topk(f32_dev(lg), k)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.moe_topk(lg, k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    wg = w.cpu().numpy().astype(np.float64)
    bound = topk_weight_bound(lg, ids_ref, k) * w_ref
    assert (np.abs(wg - w_ref) <= bound).all(), np.abs(wg - w_ref).max()


def test_topk_nan_ranks_last(gpu):
    """A NaN logit ranks as -inf: same choice as the oracle with that logit
    replaced by the lowest finite value."""
    lg = synth.router_logits(310, 64, E)
    g = synth.rng(311)
    lg[g.integers(0, 64, 40), g.integers(0, E, 40)] = np.nan
    lg[5, :] = np.nan
    lg[5, [3, 9, 17, 33, 60, 70, 90, 127]] = [1, 2, 3, 4, 5, 6, 7, 8]
    ids, w = gpu.moe_topk(f32_dev(lg), TOPK)
    torch.cuda.synchronize()
    lg_ref = np.where(np.isnan(lg), np.float32(-3.0e38), lg).astype(np.float32)
    ids_ref, w_ref = oracle.moe_topk(lg_ref, TOPK)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    assert np.isfinite(w.cpu().numpy()).all()


def test_topk_empty(gpu):
    ids, w = gpu.moe_topk(torch.empty((0, E), dtype=torch.float32, device=DEV), TOPK)
    assert ids.shape == (0, TOPK) and w.shape == (0, TOPK)


# --------------------------------------------------------------------------
# grouping by expert, row gather
# --------------------------------------------------------------------------

@pytest.mark.parametrize("tokens", [1, 5, 256, 257, 4096])
def test_permute_matches_oracle(gpu, tokens):
    _, _, ids = synth.moe_routing(320 + tokens, tokens, E, TOPK)
    off, tok, row_of = gpu.moe_permute(i32_dev(ids), E)
    torch.cuda.synchronize()
    off_r, tok_r, row_r = oracle.moe_permute(ids, E)
    np.testing.assert_array_equal(off.cpu().numpy(), off_r)
    np.testing.assert_array_equal(tok.cpu().numpy(), tok_r)
    np.testing.assert_array_equal(row_of.cpu().numpy(), row_r)


def test_permute_repeats_and_empty_experts(gpu):
    """Arbitrary ids (repeats within a token, most experts empty)."""
    g = synth.rng(330)
    ids = g.integers(0, 6, size=(700, 3)).astype(np.int32) * 20
    off, tok, row_of = gpu.moe_permute(i32_dev(ids), E)
    torch.cuda.synchronize()
    off_r, tok_r, row_r = oracle.moe_permute(ids, E)
    np.testing.assert_array_equal(off.cpu().numpy(), off_r)
    np.testing.assert_array_equal(tok.cpu().numpy(), tok_r)
    np.testing.assert_array_equal(row_of.cpu().numpy(), row_r)


def test_permute_out_of_range_ids(gpu):
    """An id outside 0..E-1 gets row -1 and no row; the other pairs keep the
    rows they have when those ids are renamed to an extra last expert."""
    _, _, ids = synth.moe_routing(331, 300, E, TOPK)
    g = synth.rng(332)
    bad = ids.copy()
    t, j = g.integers(0, 300, 50), g.integers(0, TOPK, 50)
    bad[t, j] = np.where(g.integers(0, 2, 50) == 0, -1, E + 3)
    off, tok, row_of = gpu.moe_permute(i32_dev(bad), E)
    torch.cuda.synchronize()
    renamed = np.where((bad < 0) | (bad >= E), E, bad).astype(np.int32)
    off_r, tok_r, row_r = oracle.moe_permute(renamed, E + 1)
    np.testing.assert_array_equal(off.cpu().numpy(), off_r[:E + 1])
    valid = int(off_r[E])
    np.testing.assert_array_equal(tok.cpu().numpy()[:valid], tok_r[:valid])
    ro = row_of.cpu().numpy()
    np.testing.assert_array_equal(ro, np.where(renamed == E, -1, row_r))


def test_permute_no_tokens(gpu):
    off, tok, row_of = gpu.moe_permute(torch.empty((0, TOPK), dtype=torch.int32, device=DEV), E)
    torch.cuda.synchronize()
    assert (off.cpu().numpy() == 0).all()


def test_gather_rows(gpu):
    src = synth.normal_bf16(340, (300, H))
    g = synth.rng(341)
    idx = g.integers(-5, 305, size=1001).astype(np.int32)
    out = bf16_host(gpu.gather_rows(to_dev(src), i32_dev(idx)))
    inside = (idx >= 0) & (idx < 300)
    np.testing.assert_array_equal(out[inside], src[idx[inside]])
    assert (out[~inside] == 0).all()


# --------------------------------------------------------------------------
# SwiGLU
# --------------------------------------------------------------------------

def assert_swiglu_rounding(a_bits, ref):
    """GPU bf16 = RNE(ref), except where the fp32 evaluation's error (a few
    ulps of fp32: exp, one add, one divide, one multiply) may cross a
    rounding midpoint; there either neighbour is accepted."""
    a = bf16_value(a_bits)
    # below fp32's smallest normal the fp32 evaluation underflows (for a very
    # negative gate exp(-g) is inf and silu(g) -> -0): any result that small
    tiny = np.abs(ref) < 2.0 ** -126
    assert (np.abs(a[tiny]) <= 2.0 ** -126).all(), "an underflowing output is not tiny"
    a, ref = a[~tiny], ref[~tiny]
    lo, hi = round_bf16(ref, np.floor), round_bf16(ref, np.ceil)
    assert ((a == lo) | (a == hi)).all(), "an output is not a bf16 neighbour of the fp64 value"
    rne = round_bf16(ref)
    mid = (lo + hi) / 2
    near = np.abs(ref - mid) <= 16 * U24 * np.abs(ref)
    wrong = (a != rne) & ~near
    assert not wrong.any(), "%d outputs differ from RNE away from a midpoint" % int(wrong.sum())
    return int(near.sum())


@pytest.mark.parametrize("rows,inter", [(1, 4), (37, I), (2048, I), (5, 1536)])
def test_swiglu_matches_oracle(gpu, rows, inter):
    g = synth.rng(350 + rows)
    h = (g.standard_normal((rows, 2 * inter), dtype=np.float32) * np.float32(3.0)).astype(np.float32)
    h[0, 0] = -120.0  # exp(-g) overflows to inf: silu -> -0
    a = bf16_host(gpu.swiglu(f32_dev(h)))
    ref = oracle.swiglu_f64(h)
    near = assert_swiglu_rounding(a, ref)
    assert near <= max(4, rows * inter // 1000)


# --------------------------------------------------------------------------
# weighted combine
# --------------------------------------------------------------------------

def combine_inputs(seed, tokens, k=TOPK, hidden=H):
    lg = synth.router_logits(seed, tokens, E)
    ids, w = oracle.moe_topk(lg, k)
    off, tok, row_of = oracle.moe_permute(ids, E)
    g = synth.rng(seed + 1)
    o = g.standard_normal((tokens * k, hidden), dtype=np.float32)
    return ids, w.astype(np.float32), row_of, o


def combine_fp32_ascending(o, ids, w, row_of):
    """The documented order in plain fp32 (numpy float32 is IEEE RNE): per
    token, slots by ascending expert id (stable), acc = acc + w * o."""
    t, k = ids.shape
    y = np.zeros((t, o.shape[1]), np.float32)
    for tt in range(t):
        acc = np.zeros(o.shape[1], np.float32)
        for j in np.argsort(ids[tt], kind="stable"):
            acc = (acc + (w[tt, j] * o[row_of[tt, j]]).astype(np.float32)).astype(np.float32)
        y[tt] = acc
    return y


@pytest.mark.parametrize("tokens", [1, 3, 64])
def test_combine_matches_oracle(gpu, tokens):
    ids, w, row_of, o = combine_inputs(360 + tokens, tokens)
    y = gpu.moe_combine(f32_dev(o), i32_dev(ids), f32_dev(w), i32_dev(row_of)).cpu().numpy()
    y_ref, s = oracle.moe_combine_f64(o, w, row_of)
    assert (np.abs(y - y_ref) <= (TOPK + 2) * U24 * s).all()
    ybits = y.view(np.uint32)
    emu = combine_fp32_ascending(o, ids, w, row_of)
    assert_bits_equal(ybits, emu.view(np.uint32), "combine vs fp32 sum in ascending expert id")


def test_combine_slot_order_does_not_matter(gpu):
    """Permuting a token's slots (same experts, weights and rows) keeps every
    output bit: the sum runs in expert order, not slot order."""
    ids, w, row_of, o = combine_inputs(370, 50)
    y0 = bits32(gpu.moe_combine(f32_dev(o), i32_dev(ids), f32_dev(w), i32_dev(row_of)))
    g = synth.rng(371)
    perm = np.stack([g.permutation(TOPK) for _ in range(50)])
    take = lambda a: np.take_along_axis(a, perm, axis=1)  # noqa: E731
    y1 = bits32(gpu.moe_combine(f32_dev(o), i32_dev(take(ids)), f32_dev(take(w)), i32_dev(take(row_of))))
    assert_bits_equal(y0, y1, "combine with permuted slots")


def test_combine_skips_rows_outside(gpu):
    ids, w, row_of, o = combine_inputs(372, 10)
    ro = row_of.copy()
    ro[2, 3] = -1
    ro[7, 0] = len(o) + 5
    y = gpu.moe_combine(f32_dev(o), i32_dev(ids), f32_dev(w), i32_dev(ro)).cpu().numpy()
    keep = np.ones_like(w)
    keep[2, 3] = 0
    keep[7, 0] = 0
    y_ref, s = oracle.moe_combine_f64(o, (w * keep).astype(np.float32), row_of)
    assert (np.abs(y - y_ref) <= (TOPK + 2) * U24 * s).all()


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------

MAX_TOKENS = 4096


@pytest.fixture(scope="module")
def layer(gpu):
    wr = synth.normal_bf16(380, (E, H), 0.02)
    wu = synth.normal_bf16(381, (E, 2 * I, H), 0.02)
    wd = synth.normal_bf16(382, (E, H, I), 0.02)
    dev = (to_dev(wr), to_dev(wu), to_dev(wd))
    m = gpu.MoeLayer(*dev, k=TOPK, max_tokens=MAX_TOKENS)
    return {"host": (wr, wu, wd), "dev": dev, "layer": m}


def _chain(xb, lg, lga, lg32, wu, wd, k, dl_scale):
    """Oracle steps after the router for tokens xb, whose routing is decided on
    the fp32 logits lg32, with the bound a correct fp32/bf16 implementation
    meets element by element.  lg, lga: fp64 logits and their scale
    sum |x w|; dl_scale widens the logit perturbation the weights allow."""
    ids, w = oracle.moe_topk(lg32, k)
    off, tok, row_of = oracle.moe_permute(ids, E)
    h, ha = oracle.grouped_f64(xb[tok], wu, off)
    s = oracle.swiglu_f64(h.astype(np.float32))
    a_bits = synth.f32_to_bf16_bits(round_bf16(s).astype(np.float32))
    o, oa = oracle.grouped_f64(a_bits, wd, off)
    y, ymag = oracle.moe_combine_f64(o.astype(np.float32), w.astype(np.float32), row_of)

    # h: GEMM tolerance 1e-4 * sum|x w| plus its fp32 rounding
    g, u = h[:, :I], h[:, I:]
    dh = 1e-4 * np.maximum(ha[:, :I], ha[:, I:]) + 2 * U24 * np.abs(h).max()
    # a = bf16(silu(g) u): first-order propagation of dh, a few fp32 ulps of
    # evaluation, and the two bf16 roundings (kernel and oracle) of values
    # that may straddle a midpoint
    sig = 1.0 / (1.0 + np.exp(-np.clip(g, -700, 700)))
    dsilu = np.abs(sig * (1 + g * (1 - sig)))
    ds = (dsilu * np.abs(u) + np.abs(g * sig)) * dh + 16 * U24 * np.abs(s)
    da = 2.0 ** -7 * np.abs(s) + ds * (1 + 2.0 ** -8)
    # o: da through |W_down| of the row's expert, plus the GEMM tolerance
    prop = np.zeros_like(o)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            prop[lo:hi] = da[lo:hi] @ np.abs(bf16_value(wd[e])).T
    # weights: each logit within dl of the exact one moves a weight by at most
    # a factor exp(2 dl); plus the fp32 evaluation of the softmax
    dl = 1e-4 * lga.max(axis=1) * dl_scale + 2 * U24 * np.abs(lg).max(axis=1)
    chosen = np.take_along_axis(lg32.astype(np.float64), ids.astype(np.int64), axis=1)
    dmax = np.abs(chosen - chosen[:, :1]).max(axis=1)
    dw = w * (np.expm1(2 * dl)[:, None] * 1.01 + ((k + 8 + dmax) * 2 * U24)[:, None])
    bound = np.zeros_like(y)
    for j in range(k):
        r = row_of[:, j]
        bound += np.abs(w[:, j:j + 1]) * (prop[r] + 1e-4 * oa[r] + 2 * U24 * np.abs(o[r]))
        bound += dw[:, j:j + 1] * np.abs(o[r])
    bound += (k + 4) * U24 * ymag
    return y, bound * 1.05 + 1e-30


def oracle_layer(xb, wr, wu, wd, k=TOPK):
    """The layer as a chain of oracle steps: a list, per token, of the
    (y_ref, bound) pairs a correct output may match.

    A token whose k-th and (k+1)-th logits are closer than the router GEMM's
    tolerance allows either expert set, so it gets a second pair: the chain
    with those two experts' fp32 logits swapped.
    """
    lg, lga = oracle.gemm_f64(xb, wr)
    lg32 = lg.astype(np.float32)
    y, bound = _chain(xb, lg, lga, lg32, wu, wd, k, 1.0)
    out = [[(y[t], bound[t])] for t in range(len(xb))]
    ids1, _ = oracle.moe_topk(lg32, k + 1)
    vk = np.take_along_axis(lg, ids1[:, k - 1:k].astype(np.int64), axis=1)[:, 0]
    vk1 = np.take_along_axis(lg, ids1[:, k:k + 1].astype(np.int64), axis=1)[:, 0]
    dl = 1e-4 * lga.max(axis=1)
    amb = np.nonzero(vk - vk1 <= 2 * dl + 4 * U24 * np.abs(vk))[0]
    if len(amb):
        alt = lg32[amb].copy()
        for i, t in enumerate(amb):
            ek, ek1 = int(ids1[t, k - 1]), int(ids1[t, k])
            alt[i, ek1] = np.nextafter(lg32[t, ek], np.float32(np.inf))
            alt[i, ek] = lg32[t, ek1]
        y2, b2 = _chain(xb[amb], lg[amb], lga[amb], alt, wu, wd, k, 4.0)
        for i, t in enumerate(amb):
            out[t].append((y2[i], b2[i]))
    return out, len(amb)


def run_steps(gpu, dev, x):
    """The layer's steps called one by one through the C ABI."""
    wr, wu, wd = dev
    logits = gpu.Gemm(wr)(x)
    ids, w = gpu.moe_topk(logits, TOPK)
    off, tok, row_of = gpu.moe_permute(ids, E)
    xg = gpu.gather_rows(x, tok)
    h = gpu.GroupedGemm(wu)(xg, off)
    a = gpu.swiglu(h)
    o = gpu.GroupedGemm(wd)(a, off)
    return gpu.moe_combine(o, ids, w, row_of)


@pytest.mark.parametrize("tokens", [1, 16, 256, 4096])
def test_layer_parity(gpu, layer, tokens):
    wr, wu, wd = layer["host"]
    x = synth.normal_bf16(390 + tokens, (tokens, H))
    y = layer["layer"](to_dev(x))
    torch.cuda.synchronize()
    probes = synth.probe_rows(391 + tokens, tokens, 16)
    refs, n_amb = oracle_layer(x[probes], wr, wu, wd)
    yg = y.cpu().numpy()[probes].astype(np.float64)
    err, mag = [], []
    for i, t in enumerate(probes):
        fits = [np.abs(yg[i] - yr) <= b for yr, b in refs[i]]
        if not any(f.all() for f in fits):
            f = fits[0]
            n = int(np.argmin(f))
            yr, b = refs[i][0]
            raise AssertionError("layer T=%d token %d: %d outside the bound (%d routings tried); first col %d "
                                 "gpu %r ref %r bound %r" % (tokens, t, int((~f).sum()), len(fits), n,
                                                             yg[i, n], yr[n], b[n]))
        yr = refs[i][[f.all() for f in fits].index(True)][0]
        err.append(np.abs(yg[i] - yr))
        mag.append(np.sqrt(np.mean(yr * yr)))
    # The bound above is a worst case, far above what fp32 accumulation in
    # another order gives.  Typical errors sit near fp32 rounding (about 1e-6
    # of the rms); one SwiGLU output that rounds to the other bf16 neighbour
    # moves every element of its token by about 2^-8 / sqrt(8 * 768), 5e-5 of
    # the rms.  A step done in the wrong precision (the SwiGLU output not
    # rounded to bf16, say: about 2^-9 of each term) moves the median error to
    # about 1e-3 of the rms.
    rel = np.median(np.concatenate(err)) / np.median(mag)
    print("T=%d: %d probes, %d with two admissible routings, median error %.2e of the rms"
          % (tokens, len(probes), n_amb, rel))
    assert rel <= 2.0 ** -12, "layer T=%d: median error %.3e of the rms" % (tokens, rel)


# 8 and 9 tokens sit either side of the one-launch routing and grouping;
# 16 and 17 either side of the bound on an expert's rows (a token routes to
# 8 distinct experts, so an expert has at most T rows) under which the
# streaming kernel takes every expert and applies SwiGLU in its epilogue;
# 255 and 256 either side of 16 rows per expert (8 rows a token, 128
# experts), where the four-wave kernel takes every expert and applies it
@pytest.mark.parametrize("tokens", [1, 7, 8, 9, 16, 17, 255, 256, 1024, 4096])
def test_layer_equals_its_steps(gpu, layer, tokens):
    x = to_dev(synth.normal_bf16(400 + tokens, (tokens, H)))
    y = bits32(layer["layer"](x))
    ys = bits32(run_steps(gpu, layer["dev"], x))
    assert_bits_equal(y, ys, "layer vs its steps, T=%d" % tokens)


@pytest.mark.parametrize("tokens", [16, 256, 4096])
def test_layer_batch_invariance(gpu, layer, tokens):
    """A token's output bits: alone (T = 1), inside batches of any size, at any
    position, and next to other tokens."""
    m = layer["layer"]
    x = synth.normal_bf16(410 + tokens, (tokens, H))
    y = bits32(m(to_dev(x)))
    for t in synth.probe_rows(411 + tokens, tokens, 8):
        t = int(t)
        y1 = bits32(m(to_dev(x[t:t + 1])))
        assert_bits_equal(y[t], y1[0], "token %d: T=%d vs alone" % (t, tokens))
    # shuffled batch, with a quarter of the tokens replaced by other data
    g = synth.rng(412 + tokens)
    perm = g.permutation(tokens)
    x2 = x[perm].copy()
    other = synth.normal_bf16(413 + tokens, (tokens, H))
    repl = g.random(tokens) < 0.25
    keep = ~repl[np.argsort(perm)]  # original tokens still present
    x2[repl] = other[repl]
    y2 = bits32(m(to_dev(x2)))
    inv = np.argsort(perm)
    for t in np.nonzero(keep)[0][:64]:
        assert_bits_equal(y[t], y2[inv[t]], "token %d after shuffle and co-resident change" % t)


def test_layer_edges(gpu, layer):
    m = layer["layer"]
    y = m(torch.empty((0, H), dtype=torch.bfloat16, device=DEV))
    assert y.shape == (0, H)
    with pytest.raises(gpu.BiGemmError):
        m(torch.zeros((MAX_TOKENS + 1, H), dtype=torch.bfloat16, device=DEV))
