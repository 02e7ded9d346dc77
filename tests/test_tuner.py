"""Offline pin tuner: profile parsing, legal candidates, the eq.-3 cost and
argmin, and pin-table round trips through the C library's parser (not gpu)."""
import ctypes
import os

import pytest

import invariant_bi_gemm_amd as bg
from invariant_bi_gemm_amd import tuner


def test_parse_profile():
    assert tuner.parse_profile("1:8, 16:2,4096") == [(1, 8), (16, 2), (4096, 1)]
    for bad in ("", "0:1", "4:0", "4:1,4:2"):
        with pytest.raises(ValueError):
            tuner.parse_profile(bad)


def test_legal_splits():
    assert tuner.legal_splits(14336) == [1, 2, 4, 7, 8, 14, 16]
    assert tuner.legal_splits(3584) == [1, 2, 4, 7, 8, 14]
    assert tuner.legal_splits(768) == [1, 2, 4]
    assert tuner.legal_splits(512) == [1, 2, 4, 8]
    for k in (512, 768, 2048, 3584, 4096, 14336):
        for s in tuner.legal_splits(k):
            assert k % (64 * s) == 0


def test_candidates_drop_equivalent_thresholds():
    prof = [(1, 1), (8, 1)]
    c = tuner.candidates(256, 512, prof)
    assert (1, 8) in c and (1, 16) not in c and (1, 0) in c
    assert len(c) == len(set(c))


def test_cost_and_choose():
    prof = [(1, 10), (4096, 1)]
    # synthetic timings: S = 2 is faster for M = 1 but slower at 4096
    table = {
        (1, 16): {1: 20e-6, 4096: 400e-6},
        (2, 16): {1: 15e-6, 4096: 460e-6},
        (1, 0): {1: 60e-6, 4096: 400e-6},
    }
    best, report = tuner.choose(prof, lambda c: table[c], list(table))
    assert tuner.cost(prof, table[(1, 16)]) == pytest.approx(600e-6)
    assert tuner.cost(prof, table[(2, 16)]) == pytest.approx(610e-6)
    assert best == (1, 16)
    assert len(report) == 3
    # heavier decode weight flips the choice
    prof2 = [(1, 100), (4096, 1)]
    best2, _ = tuner.choose(prof2, lambda c: table[c], list(table))
    assert best2 == (2, 16)


def test_table_round_trip_and_c_parser(tmp_path):
    path = str(tmp_path / "pins.txt")
    with open(bg.PIN_TABLE) as f:
        open(path, "w").write(f.read())
    v0, header, rows = tuner.read_table(path)
    assert rows[("gfx950", 4096, 14336)][0] >= 1 and header
    tuner.update_table(path, "gfx950", 4096, 14336, (2, 32))
    v1, header1, rows1 = tuner.read_table(path)
    assert v1 == v0 + 1 and rows1[("gfx950", 4096, 14336)] == (2, 32) and header1 == header
    assert {kk: vv for kk, vv in rows1.items() if kk != ("gfx950", 4096, 14336)} == \
           {kk: vv for kk, vv in rows.items() if kk != ("gfx950", 4096, 14336)}
    lib = bg.load()
    try:
        assert lib.bi_gemm_load_pins(path.encode()) == 0, lib.bi_last_error()
    finally:
        assert lib.bi_gemm_load_pins(bg.PIN_TABLE.encode()) == 0
    with pytest.raises(ValueError):
        tuner.update_table(path, "gfx950", 256, 512, (3, 16))  # 512 is not 3 equal parts


@pytest.mark.gpu
def test_tuner_on_device(gpu):
    """The tuner measures every legal candidate for a small layer and returns
    one of them; the chosen pin creates a working handle."""
    prof = tuner.parse_profile("1:4,24:1,200:1")
    cands = tuner.candidates(256, 512, prof, split_choices=(1, 2, 8), stream_choices=(0, 16))
    measure = tuner.device_measure(256, 512, prof, reps=3, rotate_bytes=0)
    best, report = tuner.choose(prof, measure, cands)
    assert best in cands and len(report) == len(cands)
    for _, total, t in report:
        assert total > 0 and set(t) == {1, 24, 200}
    import torch

    w = (torch.randn(256, 512, device="cuda:0") * 0.02).to(torch.bfloat16)
    g = gpu.Gemm(w, pin={"splits": best[0], "stream_max_m": best[1]})
    y = g(torch.randn(5, 512, device="cuda:0").to(torch.bfloat16))
    assert torch.isfinite(y).all()
