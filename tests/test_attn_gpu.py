"""Decode attention with a pinned split size on the GPU (gpu): parity with the
fp64 oracle within a bound derived from the kernel's tree, and batch
invariance of every request's output bits.

The bound, per output element, is (4 ds + c u) * (sum_t p_t |v_t| + |o|) with
u = 2^-24 and:
  ds = 16 u * max_t scale * sum_i |q_i k_ti|, the error of a score (four
    two-product dot instructions in order, at most two roundings each, a
    4-level butterfly, the scale in log2 units rounded once) -- also the
    error of every running or split max;
  4 ds: exp2(s - m) and the rescales exp2(m - m') each see two such errors;
  c = S/8 + splits + 32: the depth of the longest fp32 chain (a group's keys
    and its rescales, the groups and waves, the splits) plus the roundings
    of exp2 and the divide.
Shapes: Llama-3.1-8B attention (32 query heads, 8 kv heads, head dim 128) and
the other grouped-head ratios, ragged sequence lengths from 0 to 8192 keys.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, assert_bits_equal, bits32, to_dev

pytestmark = pytest.mark.gpu

U24 = 2.0 ** -24
D = 128


def make_case(seed, lengths, hq, hkv, kv_std=1.0):
    lengths = np.asarray(lengths, np.int32)
    st = np.zeros(len(lengths) + 1, np.int32)
    st[1:] = np.cumsum(lengths)
    ntok = int(st[-1])
    q = synth.normal_bf16(seed, (len(lengths), hq, D))
    k = synth.normal_bf16(seed + 1, (ntok, hkv, D), kv_std)
    v = synth.normal_bf16(seed + 2, (ntok, hkv, D))
    return q, k, v, st


def run(att, q, k, v, st):
    return att(to_dev(q), to_dev(k), to_dev(v), torch.as_tensor(st, device=DEV))


def assert_attn_parity(o_gpu, q, k, v, st, split, what, rows=None):
    scale = 1.0 / np.sqrt(D)
    o_ref, mag, qk = oracle.decode_attn_f64(q, k, v, st, scale)
    lengths = np.diff(st)
    splits = (lengths + split - 1) // split
    ds = 16 * U24 * qk
    c = split / 8 + splits[:, None] + 32
    tol = (4 * ds + c * U24)[:, :, None] * (mag + np.abs(o_ref)) + 1e-30
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    bad = err > tol
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d outside the bound; first %s gpu %r ref %r tol %r" % (
            what, int(bad.sum()), i, float(o_gpu[i]), float(o_ref[i]), float(tol[i])))


@pytest.mark.parametrize("hq,hkv,split", [(32, 8, 256), (32, 8, 512), (8, 8, 64), (16, 8, 128), (64, 8, 1024)])
def test_attn_parity_ragged(gpu, hq, hkv, split):
    lengths = [1, 5, split - 1, split, split + 1, 3 * split + 17, 0, 1000, 64]
    q, k, v, st = make_case(700 + hq + split, lengths, hq, hkv)
    att = gpu.DecodeAttention(hq, hkv, split, max_batch=16, max_seq_len=4096)
    o = run(att, q, k, v, st).cpu().numpy()
    assert_attn_parity(o, q, k, v, st, split, "Hq=%d Hkv=%d S=%d" % (hq, hkv, split))
    assert np.all(o[lengths.index(0)] == 0)


def test_attn_parity_sharp_scores(gpu):
    """Keys 4x larger: peaked softmax, scores far apart."""
    lengths = [300, 2000, 7]
    q, k, v, st = make_case(720, lengths, 32, 8, kv_std=4.0)
    att = gpu.DecodeAttention(32, 8, 256, max_batch=4, max_seq_len=4096)
    assert_attn_parity(run(att, q, k, v, st).cpu().numpy(), q, k, v, st, 256, "sharp")


def test_attn_parity_llama_decode_batch(gpu):
    """A full decode batch of 256 ragged sequences (up to 8192 keys); the
    oracle checks 16 sampled sequences."""
    lengths = synth.decode_lengths(730, 256)
    q, k, v, st = make_case(731, lengths, 32, 8)
    att = gpu.DecodeAttention(32, 8, 512, max_batch=256, max_seq_len=8192)
    o = run(att, q, k, v, st).cpu().numpy()
    for b in synth.probe_rows(732, 256, 16):
        b = int(b)
        lo, hi = int(st[b]), int(st[b + 1])
        assert_attn_parity(o[b:b + 1], q[b:b + 1], k[lo:hi], v[lo:hi], np.array([0, hi - lo], np.int32), 512,
                           "sequence %d (%d keys)" % (b, hi - lo))


def test_attn_batch_invariance(gpu):
    """Each request's bits: alone, inside a batch of 256, at another position,
    and next to other co-runners with other lengths."""
    lengths = synth.decode_lengths(740, 256)
    q, k, v, st = make_case(741, lengths, 32, 8)
    att = gpu.DecodeAttention(32, 8, 512, max_batch=256, max_seq_len=8192)
    ob = bits32(run(att, q, k, v, st))
    g = synth.rng(742)
    probes = synth.probe_rows(743, 256, 8)
    for b in probes:
        b = int(b)
        lo, hi = int(st[b]), int(st[b + 1])
        o1 = bits32(run(att, q[b:b + 1], k[lo:hi], v[lo:hi], np.array([0, hi - lo], np.int32)))
        assert_bits_equal(ob[b], o1[0], "request %d alone vs in the batch" % b)
    # a different batch: the probes shuffled among 40 other requests of other lengths
    others = synth.decode_lengths(744, 40, median=300.0)
    oq, ok, ov, _ = make_case(745, others, 32, 8)
    parts_q, parts_k, parts_v, lens, where = [], [], [], [], {}
    order = list(range(40)) + [("p", int(b)) for b in probes]
    order = [order[i] for i in g.permutation(len(order))]
    kofs = np.concatenate([[0], np.cumsum(others)])
    for item in order:
        if isinstance(item, tuple):
            b = item[1]
            lo, hi = int(st[b]), int(st[b + 1])
            where[b] = len(lens)
            parts_q.append(q[b:b + 1]), parts_k.append(k[lo:hi]), parts_v.append(v[lo:hi]), lens.append(hi - lo)
        else:
            i = item
            parts_q.append(oq[i:i + 1]), parts_k.append(ok[kofs[i]:kofs[i + 1]])
            parts_v.append(ov[kofs[i]:kofs[i + 1]]), lens.append(int(others[i]))
    st2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o2 = bits32(run(att, np.concatenate(parts_q), np.concatenate(parts_k), np.concatenate(parts_v), st2))
    for b, pos in where.items():
        assert_bits_equal(ob[b], o2[pos], "request %d in another batch at position %d" % (b, pos))


def test_attn_more_splits_than_a_wave(gpu):
    """The combine holds one split per lane of a wave: sequences of 64, 65 and
    more than 128 splits (split size 64) take its later rounds, and stay within
    the bound and invariant to the batch."""
    split = 64
    lengths = [64 * 64, 64 * 64 + 1, 9000, 3, 64 * 130 - 7]
    q, k, v, st = make_case(770, lengths, 16, 8)
    att = gpu.DecodeAttention(16, 8, split, max_batch=len(lengths), max_seq_len=9000)
    o = run(att, q, k, v, st)
    assert_attn_parity(o.cpu().numpy(), q, k, v, st, split, "up to 141 splits")
    b = 2  # 141 splits, alone
    lo, hi = int(st[b]), int(st[b + 1])
    o1 = run(att, q[b:b + 1], k[lo:hi], v[lo:hi], np.array([0, hi - lo], np.int32))
    assert_bits_equal(bits32(o)[b], bits32(o1)[0], "141 splits alone vs batch")


def test_attn_split_size_is_the_pin(gpu):
    """Two split sizes give two trees: both within the bound; one request's
    bits follow the handle's split size, not the batch."""
    lengths = [2000, 1500]
    q, k, v, st = make_case(750, lengths, 32, 8)
    for split in (256, 1024):
        att = gpu.DecodeAttention(32, 8, split, max_batch=2, max_seq_len=2048)
        o = run(att, q, k, v, st)
        assert_attn_parity(o.cpu().numpy(), q, k, v, st, split, "S=%d" % split)
        o1 = run(att, q[:1], k[:2000], v[:2000], np.array([0, 2000], np.int32))
        assert_bits_equal(bits32(o)[0], bits32(o1)[0], "S=%d alone vs batch" % split)


def test_attn_edges(gpu):
    att = gpu.DecodeAttention(32, 8, 256, max_batch=4, max_seq_len=1000)
    empty = att(torch.empty((0, 32, D), dtype=torch.bfloat16, device=DEV),
                torch.empty((0, 8, D), dtype=torch.bfloat16, device=DEV),
                torch.empty((0, 8, D), dtype=torch.bfloat16, device=DEV),
                torch.zeros(1, dtype=torch.int32, device=DEV))
    assert empty.shape == (0, 32, D)
    # a sequence longer than max_seq_len is cut there
    q, k, v, st = make_case(760, [1200, 10], 32, 8)
    o = run(att, q, k, v, st).cpu().numpy()
    st_cut = np.array([0, 1000], np.int32)
    assert_attn_parity(o[:1], q[:1], k[:1000], v[:1000], st_cut, 256, "cut at max_seq_len")
    assert_attn_parity(o[1:], q[1:], k[1200:], v[1200:], np.array([0, 10], np.int32), 256, "after a cut one")
    with pytest.raises(gpu.BiGemmError):
        att(to_dev(synth.normal_bf16(761, (5, 32, D))), to_dev(k), to_dev(v),
            torch.zeros(6, dtype=torch.int32, device=DEV))
