"""Seeded input generators (not gpu)."""
from fractions import Fraction

import numpy as np

import synth
from oracle.exact import bf16_to_fraction


def _rne_bf16_fraction(v: float) -> Fraction:
    """Nearest bf16 to v (ties to even), by exhaustive search over the two neighbours."""
    f = Fraction(float(np.float32(v)))
    bits = int(np.array([v], np.float32).view(np.uint32)[0]) >> 16
    lo, hi = bits, bits + 1 if v >= 0 else bits + 1
    cands = [bf16_to_fraction(lo), bf16_to_fraction(hi)]
    d = [abs(c - f) for c in cands]
    if d[0] != d[1]:
        return cands[int(d[1] < d[0])]
    return cands[0] if (lo & 1) == 0 else cands[1]


def test_bf16_round_to_nearest_even():
    g = synth.rng(5)
    vals = np.concatenate([
        g.standard_normal(2000).astype(np.float32),
        np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 3.0, -0.0, 65504.0, 1e-3], np.float32),
    ])
    bits = synth.f32_to_bf16_bits(vals)
    for v, b in zip(vals, bits):
        assert bf16_to_fraction(int(b)) == _rne_bf16_fraction(float(v)), v
    assert np.array_equal(synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(bits)), bits)


def test_same_seed_same_bits():
    assert np.array_equal(synth.normal_bf16(42, (64, 128)), synth.normal_bf16(42, (64, 128)))
    assert not np.array_equal(synth.normal_bf16(42, (64, 128)), synth.normal_bf16(43, (64, 128)))
    assert np.array_equal(synth.silu_mul_bf16(7, (4, 32)), synth.silu_mul_bf16(7, (4, 32)))


def test_distributions():
    w = synth.bf16_bits_to_f32(synth.normal_bf16(42, (256, 512), 0.02))
    assert abs(w.std() - 0.02) < 0.001 and abs(w.mean()) < 0.001
    i = synth.bf16_bits_to_f32(synth.int_bf16(1, (100, 100)))
    assert set(np.unique(i).tolist()) == set(range(-3, 4))
    r = synth.bf16_bits_to_f32(synth.rms_rows_bf16(2, (16, 4096)))
    rms = np.sqrt((r.astype(np.float64) ** 2).mean(axis=1))
    assert np.all(np.abs(rms - 1) < 0.01)
    s = synth.bf16_bits_to_f32(synth.silu_mul_bf16(3, (64, 1024)))
    assert np.isfinite(s).all() and 0.3 < s.std() < 1.5


def test_moe_routing_tables():
    tok, off, ids = synth.moe_routing(42, 256, experts=128, topk=8)
    assert off[0] == 0 and off[-1] == 256 * 8 and np.all(np.diff(off) >= 0)
    for t in range(256):
        assert len(set(ids[t].tolist())) == 8
    # each expert's rows are its tokens, ascending
    for e in range(128):
        rows = tok[off[e]:off[e + 1]]
        assert np.all(np.diff(rows) > 0)
        for t in rows:
            assert e in ids[t]
    # every expert is about equally popular (uniform 8-subsets: 16 rows each)
    counts = np.diff(off)
    assert counts.min() > 0 and abs(counts.mean() - 16) < 1e-9 and counts.max() < 48
    # same seed, same routing
    tok2, off2, ids2 = synth.moe_routing(42, 256, experts=128, topk=8)
    assert np.array_equal(tok, tok2) and np.array_equal(off, off2) and np.array_equal(ids, ids2)


def test_router_logits():
    lg = synth.router_logits(5, 64, 128)
    assert lg.dtype == np.float32 and lg.shape == (64, 128) and 0.8 < lg.std() < 1.2
    q = synth.router_logits(5, 64, 128, step=0.25)
    assert np.all(q * 4 == np.round(q * 4))
    # rounding makes ties common
    assert any(len(set(row.tolist())) < 128 for row in q)


def test_probe_rows():
    assert np.array_equal(synth.probe_rows(1, 10), np.arange(10))
    p = synth.probe_rows(1, 8192)
    assert p.size == 64 and len(set(p.tolist())) == 64 and p.max() < 8192
    assert np.array_equal(p, synth.probe_rows(1, 8192))
