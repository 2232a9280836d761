"""Pins for the reference tile schedule (oracle/schedule.py).

Fixed independently of the oracle by: the hand-worked schedule of the 512^3
shape (tests/golden/schedule_cfg1.txt), the page's printed manual-walk formula
(page "[Feature] Introduce tile scheduler #2441", gemm_persistent's removed
tile walk) wherever its own assertion n_blocks % group_size == 0 holds, and
invariants any persistent grid-strided schedule must satisfy.
"""

import itertools
import os

import pytest

from oracle import schedule as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page_walk(tile_id, m_blocks, group_size):
    # the formula as printed in the removed manual walk
    bx = (tile_id // group_size) % m_blocks
    by = tile_id % group_size + (tile_id // group_size) // m_blocks * group_size
    return bx, by


def test_golden_cfg1_table():
    rows = []
    with open(os.path.join(GOLDEN, "schedule_cfg1.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append(tuple(int(v) for v in line.split()))
    assert S.schedule(8, 4, 4, 2) == rows


SWEEP = [(m, n, gs, P) for m in range(1, 9) for n in range(1, 13) for gs in (1, 2, 3, 4, 5, 8, 13)
         for P in (1, 3, 8)]


@pytest.mark.parametrize("m_blocks,n_blocks,gs,P", [c for c in SWEEP if c[1] % c[2] == 0])
def test_matches_page_walk_when_groups_are_full(m_blocks, n_blocks, gs, P):
    for w, wid in itertools.product(range(m_blocks * n_blocks // P + 2), range(P)):
        t = P * w + wid
        if t < m_blocks * n_blocks:
            assert S.coord(t, m_blocks, n_blocks, gs) == _page_walk(t, m_blocks, gs)
            bx, by = _page_walk(t, m_blocks, gs)
            assert bx < m_blocks and by < n_blocks          # the page's guard holds
        else:
            _, by = _page_walk(t, m_blocks, gs)
            assert by >= n_blocks                           # guard fails exactly past the end


@pytest.mark.parametrize("m_blocks,n_blocks,gs,P", SWEEP[::3])
def test_invariants(m_blocks, n_blocks, gs, P):
    rows = S.schedule(P, m_blocks, n_blocks, gs)
    T = m_blocks * n_blocks
    assert len(rows) == T
    assert sorted((m, n) for _, _, m, n in rows) == [(m, n) for m in range(m_blocks) for n in range(n_blocks)]
    for wid in range(P):
        mine = [r for r in rows if r[0] == wid]
        assert len(mine) == max(0, -(-(T - wid) // P))
        assert [r[1] for r in mine] == list(range(len(mine)))
        assert mine == sorted(mine)
    # (worker, iter) -> tile id P*iter + worker, and decode agrees
    for wid, it, m, n in rows:
        assert S.coord(P * it + wid, m_blocks, n_blocks, gs) == (m, n)
    assert rows == sorted(rows)


def test_page_walk_breaks_on_partial_group():
    """m_blocks=3, n_blocks=5, group_size=2 violates the page's assertion; its walk
    would visit column 5 (absent) and miss (2, 4).  The oracle's partial last
    group covers every tile once."""
    visited = {_page_walk(t, 3, 2) for t in range(15)}
    assert (0, 5) in visited and (2, 4) not in visited
    rows = S.schedule(4, 3, 5, 2)
    assert sorted((m, n) for _, _, m, n in rows) == [(m, n) for m in range(3) for n in range(5)]


def test_group_wider_than_grid_is_row_major():
    rows = S.schedule(1, 3, 4, 99)
    assert [(m, n) for _, _, m, n in rows] == [(m, n) for m in range(3) for n in range(4)]


def test_more_workers_than_tiles():
    rows = S.schedule(256, 8, 8, 4)
    assert len(rows) == 64 and all(it == 0 for _, it, _, _ in rows)
    assert [r[0] for r in rows] == list(range(64))


# ---------------------------------------------------------------- scheduler options
def _page_walk_2cta(block_id, w, P, m_blocks, group_size):
    # the 2-CTA manual walk as printed (removed side of gemm_persistent_2cta):
    # num_clusters = sm_num // 2, m_clusters = m_blocks // 2
    num_clusters, m_clusters = P // 2, m_blocks // 2
    cluster_id, cta_id = block_id // 2, block_id % 2
    tile_id = num_clusters * w + cluster_id
    bx_cluster = (tile_id // group_size) % m_clusters
    bx = bx_cluster * 2 + cta_id
    by = (tile_id % group_size) + (tile_id // group_size) // m_clusters * group_size
    return bx, by


CLUSTER_SWEEP = [(m, n, gs, P) for m in (2, 4, 6, 8) for n in range(1, 13) for gs in (1, 2, 3, 4, 6)
                 for P in (2, 4, 6, 16) if n % gs == 0]


@pytest.mark.parametrize("m_blocks,n_blocks,gs,P", CLUSTER_SWEEP[::2])
def test_cluster_two_matches_page_2cta_walk(m_blocks, n_blocks, gs, P):
    """Where the page's walk is defined (m_blocks even, full column groups),
    cluster_size=2 visits exactly the tiles the printed walk visits, on the same
    workgroup and wave; the walk's own bounds guard ends each workgroup's run."""
    rows = S.schedule(P, m_blocks, n_blocks, gs, cluster_size=2)
    want = []
    waves = m_blocks * n_blocks // P + 2
    for block_id in range(P):
        for w in range(waves):
            bx, by = _page_walk_2cta(block_id, w, P, m_blocks, gs)
            if bx < m_blocks and by < n_blocks:
                want.append((block_id, w, bx, by))
    assert rows == sorted(want)


@pytest.mark.parametrize("m_blocks,n_blocks,gs,P", SWEEP[::5])
def test_cluster_one_and_row_major_are_the_default(m_blocks, n_blocks, gs, P):
    assert S.schedule(P, m_blocks, n_blocks, gs, column_major=False, cluster_size=1) == \
        S.schedule(P, m_blocks, n_blocks, gs)


@pytest.mark.parametrize("m_blocks,n_blocks,gs,P", SWEEP[::5])
def test_column_major_is_the_transposed_walk(m_blocks, n_blocks, gs, P):
    """Column-major on an m x n grid = the default walk of the n x m grid with
    the coordinates swapped back."""
    t = S.schedule(P, n_blocks, m_blocks, gs)
    assert S.schedule(P, m_blocks, n_blocks, gs, column_major=True) == [(w, i, b, a) for w, i, a, b in t]
    # with one group spanning every row block, column-major walks the grid
    # column by column, m fastest (the default walks it row by row)
    rows = S.schedule(1, m_blocks, n_blocks, m_blocks, column_major=True)
    assert [(m, n) for _, _, m, n in rows] == [(m, n) for n in range(n_blocks) for m in range(m_blocks)]
    rows = S.schedule(1, m_blocks, n_blocks, n_blocks)
    assert [(m, n) for _, _, m, n in rows] == [(m, n) for m in range(m_blocks) for n in range(n_blocks)]


@pytest.mark.parametrize("cs", [1, 2, 3, 4])
@pytest.mark.parametrize("cm", [False, True])
def test_option_invariants(cs, cm):
    for m_blocks, n_blocks, gs, mult in itertools.product((1, 2, 3, 5, 7), (1, 3, 4), (1, 2, 5), (1, 2, 3)):
        P = cs * mult
        rows = S.schedule(P, m_blocks, n_blocks, gs, column_major=cm, cluster_size=cs)
        # every tile once
        assert sorted((m, n) for _, _, m, n in rows) == [(m, n) for m in range(m_blocks) for n in range(n_blocks)]
        m_cl = -(-m_blocks // cs)
        for wid in range(P):
            mine = [r for r in rows if r[0] == wid]
            its = [r[1] for r in mine]
            assert its == sorted(set(its))                       # waves strictly increase
            assert all(r[2] % cs == wid % cs for r in mine)       # rank picks the row inside the cluster
            # the cluster's wave count, minus the waves whose row block does not exist
            clusters = P // cs
            waves = max(0, -(-(m_cl * n_blocks - wid // cs) // clusters))
            skipped = sum(1 for w in range(waves)
                          if S.coord(clusters * w + wid // cs, m_cl, n_blocks, gs, cm)[0] * cs + wid % cs >= m_blocks)
            assert len(mine) == waves - skipped


def test_cluster_needs_whole_clusters():
    with pytest.raises(ValueError):
        S.schedule(5, 4, 4, 2, cluster_size=2)
