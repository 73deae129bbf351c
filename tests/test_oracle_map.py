"""Pins of the oracle's block -> tile map against things other than itself.

Sources ("Block Scheduler Code Explained", CATLASS docs): loop counts s4.1 /
s4.3, batch index s4.4, Zn windows + snake s4.5 / s5.1 / s5.2, tail shapes
s4.6 / s5.3, runtime offset and direction s6.  The pins:
  * a generative enumeration written from the prose description of the
    windows (not from the index arithmetic the oracle transcribes);
  * bijection over all tiles and tail sums (s4.6: the tail tiles fill the
    problem exactly);
  * special cases with a closed form (offset 1 = boustrophedon rows, one
    window = column-major, Nz with one window = row-major raster);
  * the hand-derived worked example in tests/golden/tails_map_zn3.txt.
The Nz branch is elided on the page; its mirror reading is checked for
self-consistency (Nz == transposed Zn) only: parity unpinned as to the
reading itself.
"""
import itertools
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def cdiv(a, b):
    return -(-a // b)


def enumerate_zn(loopsM, loopsN, off):
    """Windows of `off` tile-rows, walked in order; inside a window, column
    by column (reversed on odd windows), and inside a column the window's
    rows top to bottom."""
    seq = []
    for w in range(cdiv(loopsM, off)):
        rows = range(w * off, min((w + 1) * off, loopsM))
        cols = range(loopsN) if w % 2 == 0 else range(loopsN - 1, -1, -1)
        for n in cols:
            for m in rows:
                seq.append((m, n))
    return seq


def enumerate_nz(loopsM, loopsN, off):
    """Windows of `off` tile-columns; inside a window row by row (reversed
    on odd windows), and inside a row the window's columns left to right."""
    seq = []
    for w in range(cdiv(loopsN, off)):
        cols = range(w * off, min((w + 1) * off, loopsN))
        rows = range(loopsM) if w % 2 == 0 else range(loopsM - 1, -1, -1)
        for m in rows:
            for n in cols:
                seq.append((m, n))
    return seq


SHAPES = [(1, 1, 1, 1), (200, 136, 64, 64), (1024, 1024, 256, 128), (1000, 700, 64, 32),
          (64, 640, 64, 64), (640, 64, 64, 64), (7, 13, 2, 3), (300, 500, 128, 128),
          (1, 999, 16, 16), (999, 1, 16, 16), (96, 96, 32, 32)]
OFFSETS = [1, 2, 3, 4, 5, 8, 1000]


@pytest.mark.parametrize("M,N,tm,tn", SHAPES)
@pytest.mark.parametrize("off", OFFSETS)
def test_zn_and_nz_match_generative_enumeration(orc, M, N, tm, tn, off):
    lm, ln = cdiv(M, tm), cdiv(N, tn)
    zn = orc.tile_map(1, M, N, tm, tn, off, "zn")
    assert [tuple(r) for r in zn[:, 1:3].tolist()] == enumerate_zn(lm, ln, off)
    nz = orc.tile_map(1, M, N, tm, tn, off, "nz")
    assert [tuple(r) for r in nz[:, 1:3].tolist()] == enumerate_nz(lm, ln, off)


@pytest.mark.parametrize("M,N,tm,tn", SHAPES)
@pytest.mark.parametrize("off", OFFSETS)
@pytest.mark.parametrize("direction", ["zn", "nz", "raster"])
def test_bijection_and_tail_shapes(orc, M, N, tm, tn, off, direction):
    lm, ln = cdiv(M, tm), cdiv(N, tn)
    mp = orc.tile_map(1, M, N, tm, tn, off, direction)
    assert mp.shape == (lm * ln, 5)
    tiles = {(int(m), int(n)) for m, n in mp[:, 1:3]}
    assert tiles == set(itertools.product(range(lm), range(ln)))
    # tail shapes: every tile is full except the last tile-row / column, and
    # the actual extents of one tile-column (row) add up to M (N).
    act = {(int(r[1]), int(r[2])): (int(r[3]), int(r[4])) for r in mp}
    assert sum(act[(m, 0)][0] for m in range(lm)) == M
    assert sum(act[(0, n)][1] for n in range(ln)) == N
    for (m, n), (ma, na) in act.items():
        assert ma == (tm if m < lm - 1 else M - (lm - 1) * tm)
        assert na == (tn if n < ln - 1 else N - (ln - 1) * tn)
        assert 1 <= ma <= tm and 1 <= na <= tn


def test_special_cases(orc):
    lm, ln = 6, 5
    M, N = lm * 16, ln * 16
    # offset 1: one tile-row per window, odd rows reversed (boustrophedon)
    zn1 = orc.tile_map(1, M, N, 16, 16, 1, "zn")[:, 1:3].tolist()
    expect = [[m, n if m % 2 == 0 else ln - 1 - n] for m in range(lm) for n in range(ln)]
    assert zn1 == expect
    # one Zn window covering all tile-rows: column-major order, no reversal
    znall = orc.tile_map(1, M, N, 16, 16, lm, "zn")[:, 1:3].tolist()
    assert znall == [[m, n] for n in range(ln) for m in range(lm)]
    # one Nz window covering all tile-columns == row-major RASTER
    nzall = orc.tile_map(1, M, N, 16, 16, ln, "nz")[:, 1:3].tolist()
    raster = orc.tile_map(1, M, N, 16, 16, 1, "raster")[:, 1:3].tolist()
    assert nzall == raster == [[m, n] for m in range(lm) for n in range(ln)]
    # an offset beyond the tile count behaves as one window
    assert orc.tile_map(1, M, N, 16, 16, 1000, "zn").tolist() == \
        orc.tile_map(1, M, N, 16, 16, lm, "zn").tolist()


@pytest.mark.parametrize("M,N,tm,tn", SHAPES)
@pytest.mark.parametrize("off", [1, 2, 3, 7])
def test_nz_is_transposed_zn(orc, M, N, tm, tn, off):
    nz = orc.tile_map(1, M, N, tm, tn, off, "nz")
    zn_t = orc.tile_map(1, N, M, tn, tm, off, "zn")
    assert np.array_equal(nz[:, 1], zn_t[:, 2]) and np.array_equal(nz[:, 2], zn_t[:, 1])
    assert np.array_equal(nz[:, 3], zn_t[:, 4]) and np.array_equal(nz[:, 4], zn_t[:, 3])


def test_batch_index(orc):
    M, N, tm, tn, batch = 100, 70, 32, 32, 5
    core = cdiv(M, tm) * cdiv(N, tn)
    mp = orc.tile_map(batch, M, N, tm, tn, 2, "zn")
    assert mp.shape[0] == batch * core
    assert np.array_equal(mp[:, 0], np.arange(batch * core) // core)
    one = orc.tile_map(1, M, N, tm, tn, 2, "zn")
    for b in range(batch):
        assert np.array_equal(mp[b * core:(b + 1) * core, 1:], one[:, 1:])


def test_worked_example_tails(orc):
    rows = [list(map(int, ln.split())) for ln in open(os.path.join(GOLDEN, "tails_map_zn3.txt"))
            if ln.strip() and not ln.startswith("#")]
    expect = np.array([r[1:] for r in rows], np.uint32)
    assert [r[0] for r in rows] == list(range(12))
    got = orc.tile_map(1, 200, 136, 64, 64, 3, "zn")
    assert np.array_equal(got, expect)


def test_empty_problems(orc):
    assert orc.tile_map(1, 0, 100, 64, 64, 1, "zn").shape[0] == 0
    assert orc.tile_map(1, 100, 0, 64, 64, 1, "nz").shape[0] == 0
    assert orc.tile_map(0, 100, 100, 64, 64, 1, "zn").shape[0] == 0
    with pytest.raises(ValueError):
        orc.tile_map(1, 10, 10, 4, 4, 0, "zn")       # offset 0 is undefined
    with pytest.raises(ValueError):
        orc.tile_map(1, 10, 10, 4, 4, 1, 3)          # no such direction


@pytest.mark.parametrize("direction", ["zn", "nz", "raster"])
def test_grouped_map_is_concatenation(orc, direction):
    gm = [0, 300, 5, 0, 129, 64, 1]
    N, tm, tn, off = 200, 64, 64, 2
    mp = orc.grouped_tile_map(gm, N, tm, tn, off, direction)
    t, row0 = 0, 0
    for g, Mg in enumerate(gm):
        one = orc.tile_map(1, Mg, N, tm, tn, off, direction)
        part = mp[t:t + one.shape[0]]
        assert np.all(part[:, 0] == g)
        assert np.array_equal(part[:, 1:5], one[:, 1:5])
        assert np.array_equal(part[:, 5], row0 + one[:, 1] * tm)
        t += one.shape[0]
        row0 += Mg
    assert t == mp.shape[0]
