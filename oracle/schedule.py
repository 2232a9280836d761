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

Rows are (worker, iter, m_idx, n_idx) sorted by (worker, iter).
"""

from __future__ import annotations


def coord(tile_id: int, m_blocks: int, n_blocks: int, group_size: int) -> tuple[int, int]:
    """Stateless decode of one linear tile id into (m_idx, n_idx).

    Column groups of ``group_size`` n-blocks are walked in order; inside a group
    the tiles are laid out row after row (m slow, n fast), each row being as
    wide as the group.
    """
    per_group = group_size * m_blocks
    group = tile_id // per_group
    first_col = group * group_size
    width = min(group_size, n_blocks - first_col)
    r = tile_id - group * per_group
    return r // width, first_col + r % width


def schedule_closed_form(num_workers: int, m_blocks: int, n_blocks: int,
                         group_size: int) -> list[tuple[int, int, int, int]]:
    """Worker-major enumeration driven by the wave clock.

    For each worker: start at wave 0, visit tile ``num_workers * w + worker``
    while it is below the tile count, then advance the wave index.
    """
    tiles = m_blocks * n_blocks
    rows = []
    for worker in range(num_workers):
        w = 0
        while num_workers * w + worker < tiles:
            m, n = coord(num_workers * w + worker, m_blocks, n_blocks, group_size)
            rows.append((worker, w, m, n))
            w += 1
    return rows


def schedule_by_walk(num_workers: int, m_blocks: int, n_blocks: int,
                     group_size: int) -> list[tuple[int, int, int, int]]:
    """Second, independent construction of the same schedule.

    First write down the global visiting order by walking the column groups,
    then the rows inside a group, then the columns of the group; then deal the
    ordered list round-robin: item i goes to worker i % P at wave i // P.
    """
    order = []
    for first_col in range(0, n_blocks, group_size):
        cols = list(range(first_col, min(first_col + group_size, n_blocks)))
        for m in range(m_blocks):
            for n in cols:
                order.append((m, n))
    dealt = [(i % num_workers, i // num_workers, m, n) for i, (m, n) in enumerate(order)]
    return sorted(dealt)


def schedule(num_workers: int, m_blocks: int, n_blocks: int, group_size: int):
    """The reference schedule; both constructions must agree."""
    a = schedule_closed_form(num_workers, m_blocks, n_blocks, group_size)
    b = schedule_by_walk(num_workers, m_blocks, n_blocks, group_size)
    if a != b:
        raise AssertionError("schedule constructions disagree")
    return a
