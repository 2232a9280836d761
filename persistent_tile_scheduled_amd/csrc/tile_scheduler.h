// Persistent tile scheduler, compiled both for the host and for gfx950.
//
// Page "[Feature] Introduce tile scheduler #2441" (diff of
// examples/gemm_sm100/gemm_tcgen5mma_ws_persistent.py): each warp role builds
// its own PersistentTileScheduler, calls init(block_id), loops while valid()
// and advances with next_tile(); the scheduler's current_iter is the wave index
// w and m_idx / n_idx are the tile coordinates.  (The page selects one of two
// TMEM accumulators by w & 1; the kernels here keep one accumulator set per
// wave, and `iter` is exported through the schedule dump and the kernel's
// trace.)  The removed manual walk it replaces gives worker `wid` the
// linear tiles P*w + wid and decodes them in groups of group_size column
// blocks, rows of the group walked one after the other.  The conversation tab
// describes a stateless coord(tile_id) next to the stateful iteration.
//
// Here every wavefront keeps its own copy in scalar registers (all members are
// wave-uniform), the loader and the MMA loop each hold one, as the page's
// roles do, and no coordinates are exchanged between them.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define TSG_HD __host__ __device__ __forceinline__
#else
#define TSG_HD inline
#endif

namespace tsg {

struct TileScheduler {
    uint32_t num_workers;  // clusters: P / cluster
    uint32_t m_blocks, n_blocks, group, cluster, col_major;
    uint32_t m_cl;         // cluster rows: ceil(m_blocks / cluster)
    uint32_t tiles;        // cluster tiles: m_cl * n_blocks
    uint32_t rank, iter, tile_id;
    uint32_t m_idx, n_idx;

    // P workgroups in clusters of cs (P % cs == 0), decode column groups of gs
    // blocks (cm = 0) or its transpose, row groups of gs blocks (cm = 1).
    TSG_HD void setup(uint32_t P, uint32_t mb, uint32_t nb, uint32_t gs, uint32_t cs = 1, uint32_t cm = 0) {
        cluster = cs;
        col_major = cm;
        num_workers = P / cs;
        m_blocks = mb;
        n_blocks = nb;
        group = gs;
        m_cl = (mb + cs - 1) / cs;
        tiles = m_cl * nb;
    }

    // Decode one linear cluster-tile id on the m_cl x n_blocks grid.  Row-major:
    // column group g covers n blocks [g*group, g*group + width), width = group
    // except a narrower last group; inside the group tiles run row by row.
    // Column-major: the same walk with the roles of rows and columns swapped.
    TSG_HD void coord(uint32_t t, uint32_t& m, uint32_t& n) const {
        const uint32_t rows = col_major ? n_blocks : m_cl;
        const uint32_t cols = col_major ? m_cl : n_blocks;
        const uint32_t per_group = group * rows;
        const uint32_t g = t / per_group;
        const uint32_t first = g * group;
        const uint32_t rest = cols - first;
        const uint32_t width = rest < group ? rest : group;
        const uint32_t r = t - g * per_group;
        const uint32_t row = r / width;
        const uint32_t col = first + (r - row * width);
        m = col_major ? col : row;
        n = col_major ? row : col;
    }

    // Workgroup wid is rank wid % cluster of cluster wid / cluster; the cluster
    // visits tile ids cluster_id + num_workers * iter.
    TSG_HD void init(uint32_t wid) {
        const uint32_t c = wid / cluster;
        rank = wid - c * cluster;
        iter = 0;
        tile_id = c;
        update();
    }
    TSG_HD bool valid() const { return tile_id < tiles; }
    TSG_HD void next_tile() {
        ++iter;
        tile_id += num_workers;
        update();
    }

  private:
    // The workgroup takes row block m * cluster + rank of its cluster's tile;
    // a rank whose row block is past the last one skips that wave.
    TSG_HD void update() {
        while (valid()) {
            uint32_t m, n;
            coord(tile_id, m, n);
            const uint32_t bx = m * cluster + rank;
            if (bx < m_blocks) {
                m_idx = bx;
                n_idx = n;
                return;
            }
            ++iter;
            tile_id += num_workers;
        }
    }
};

// Hardware hands workgroups to the XCDs round robin (workgroup b runs on XCD
// b % X).  Renumber them so that each XCD holds contiguous runs of worker ids:
// consecutive tile ids, hence a compact block of one column group, then share
// that XCD's L2.  Only the first A worker ids have tiles when the tile count
// is below the worker count, so those are split evenly over the XCDs (XCD x
// gets active ids [x*qa + min(x, ra), ...) with qa = A / X, ra = A % X) and the
// idle ids fill the remaining slots; with A = P every XCD simply gets one run.
// A bijection on [0, P) for every P, X >= 1 and 1 <= A <= P.
TSG_HD uint32_t worker_of_workgroup(uint32_t b, uint32_t P, uint32_t X, uint32_t A) {
    if (X <= 1u) return b;
    const uint32_t x = b % X, j = b / X;
    const uint32_t q = P / X, r = P % X;      // XCD x holds q + (x < r) workgroups
    const uint32_t qa = A / X, ra = A % X;    // ... of which qa + (x < ra) are active
    const uint32_t active_x = qa + (x < ra ? 1u : 0u);
    const uint32_t first_active = x * qa + (x < ra ? x : ra);
    if (j < active_x) return first_active + j;
    const uint32_t first_slot = x * q + (x < r ? x : r);
    return A + (first_slot - first_active) + (j - active_x);
}

}  // namespace tsg
