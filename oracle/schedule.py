"""Reference enumeration of the persistent tile schedule -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use this
module.  It shares no code with the HIP path.

Source: page "[Feature] Introduce tile scheduler #2441", diff of
examples/gemm_sm100/gemm_tcgen5mma_ws_persistent.py, function gemm_persistent.
The removed manual walk gives worker ``block_id`` the tiles
``tile_id = sm_num * w + block_id`` for wave index ``w`` and decodes them in
groups of ``group_size`` column blocks (m index cycles over all row blocks
inside a group, n index is fast within the group); the added
``PersistentTileScheduler(..., swizzle_size=group_size)`` replaces that walk and
keeps the wave index as ``current_iter``.  The page's conversation tab (PR
overview of tile_schedule.py) lists the scheduler's init / valid / next_tile
and a stateless ``coord(tile_id)`` decode.

Readings taken where the pages are silent:
  * valid() is ``tile_id < m_blocks * n_blocks`` (the page's new loop has no
    bounds guard; with the page's own assertion n_blocks % group_size == 0 the
    two agree).
  * When n_blocks is not a multiple of group_size the last column group is
    narrower (``width = min(gs, n_blocks - first_col)``); with a full last group
    this is the page's formula unchanged.
  * The number of workers is the number of persistent workgroups (the page uses
    the SM count with one CTA per worker).

Two scheduler options named in the PR overview on the same page
(PersistentTileScheduler's cluster_size and column_major), read as follows:
  * cluster_size = cs (the 2-CTA variant gemm_persistent_2cta): workgroup
    ``wid`` belongs to cluster ``wid // cs`` with rank ``cta = wid % cs``; the
    scheduler runs over ``P // cs`` clusters (init(block_id // cluster_size))
    on a grid of ``ceil(m_blocks / cs)`` cluster rows by n_blocks, and the
    workgroup takes row block ``bx = m_idx * cs + cta``, column ``n_idx``.  When
    m_blocks is not a multiple of cs the tail cluster's bx can pass the last row
    block; the review on the page asks for a ``bx < m_blocks`` guard, read here
    as: that workgroup skips the iteration (no tile, the wave index still
    advances).  P must be a multiple of cs.
  * column_major: the page gives only "axis fast/slow selection".  Read as the
    transpose of the default decode: groups of group_size row blocks, and inside
    a group the tiles run column by column (n slow, m fast).

Rows are (worker, iter, m_idx, n_idx) sorted by (worker, iter).
"""

from __future__ import annotations


def coord(tile_id: int, m_blocks: int, n_blocks: int, group_size: int,
          column_major: bool = False) -> tuple[int, int]:
    """Stateless decode of one linear tile id into (m_idx, n_idx).

    Column groups of ``group_size`` n-blocks are walked in order; inside a group
    the tiles are laid out row after row (m slow, n fast), each row being as
    wide as the group.  ``column_major`` swaps the roles of m and n.
    """
    if column_major:
        n, m = coord(tile_id, n_blocks, m_blocks, group_size)
        return m, n
    per_group = group_size * m_blocks
    group = tile_id // per_group
    first_col = group * group_size
    width = min(group_size, n_blocks - first_col)
    r = tile_id - group * per_group
    return r // width, first_col + r % width


def _cluster_grid(num_workers: int, m_blocks: int, cluster_size: int):
    if cluster_size < 1 or num_workers % cluster_size:
        raise ValueError("the number of workers must be a multiple of cluster_size")
    return num_workers // cluster_size, -(-m_blocks // cluster_size)


def schedule_closed_form(num_workers: int, m_blocks: int, n_blocks: int, group_size: int,
                         column_major: bool = False, cluster_size: int = 1
                         ) -> list[tuple[int, int, int, int]]:
    """Worker-major enumeration driven by the wave clock.

    For each worker: start at wave 0, visit cluster tile ``clusters * w +
    cluster`` while it is below the cluster-tile count, take row block
    ``m * cs + cta`` of it when that block exists, then advance the wave index.
    """
    clusters, m_cl = _cluster_grid(num_workers, m_blocks, cluster_size)
    tiles = m_cl * n_blocks
    rows = []
    for worker in range(num_workers):
        cluster, cta = divmod(worker, cluster_size)
        w = 0
        while clusters * w + cluster < tiles:
            m, n = coord(clusters * w + cluster, m_cl, n_blocks, group_size, column_major)
            bx = m * cluster_size + cta
            if bx < m_blocks:
                rows.append((worker, w, bx, n))
            w += 1
    return rows


def schedule_by_walk(num_workers: int, m_blocks: int, n_blocks: int, group_size: int,
                     column_major: bool = False, cluster_size: int = 1
                     ) -> list[tuple[int, int, int, int]]:
    """Second, independent construction of the same schedule.

    First write down the global visiting order of cluster tiles by walking the
    groups, then the rows (columns, if column-major) inside a group, then the
    other axis within the group; deal the ordered list round-robin to the
    clusters (item i to cluster i % C at wave i // C); finally split every
    cluster tile into its cs row blocks, one per rank, dropping blocks past the
    last row.
    """
    clusters, m_cl = _cluster_grid(num_workers, m_blocks, cluster_size)
    order = []
    if not column_major:
        for first_col in range(0, n_blocks, group_size):
            cols = list(range(first_col, min(first_col + group_size, n_blocks)))
            for m in range(m_cl):
                for n in cols:
                    order.append((m, n))
    else:
        for first_row in range(0, m_cl, group_size):
            rws = list(range(first_row, min(first_row + group_size, m_cl)))
            for n in range(n_blocks):
                for m in rws:
                    order.append((m, n))
    dealt = []
    for i, (m, n) in enumerate(order):
        cluster, w = i % clusters, i // clusters
        for cta in range(cluster_size):
            if m * cluster_size + cta < m_blocks:
                dealt.append((cluster * cluster_size + cta, w, m * cluster_size + cta, n))
    return sorted(dealt)


def schedule(num_workers: int, m_blocks: int, n_blocks: int, group_size: int,
             column_major: bool = False, cluster_size: int = 1):
    """The reference schedule; both constructions must agree."""
    a = schedule_closed_form(num_workers, m_blocks, n_blocks, group_size, column_major, cluster_size)
    b = schedule_by_walk(num_workers, m_blocks, n_blocks, group_size, column_major, cluster_size)
    if a != b:
        raise AssertionError("schedule constructions disagree")
    return a
