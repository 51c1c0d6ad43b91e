// Work decomposition shared by the host planner and the gfx950 kernel.
//
// Everything here is integer arithmetic on tile and iteration indices.  The
// same inline functions run on the host (planning, introspection, the
// coverage tests) and inside the kernel, so what the tests check is what the
// GPU executes.
//
// Vocabulary (Triton issue #1393 "Stream-k matmul implementation very
// slow...", final revision):
//   T      output tiles, tiles_m * tiles_n
//   ipt    MAC iterations per tile, ceil(K / bk)
//   g      workgroups of the Stream-K / persistent launch
//   T_sk   tiles [0, T_sk) whose iterations are spread over the g workgroups
//   q, r   T_sk * ipt = q * g + r; workgroup p owns iterations
//          [p*q + min(p, r), (p+1)*q + min(p+1, r))
// With a per-tile split (sk_split = s > 0, not on the pages) each Stream-K
// tile t is instead cut into s pieces by the same rule, ipt = q * s + r:
// workgroup p = t*s + j owns iterations t*ipt + [j*q + min(j, r),
// (j+1)*q + min(j+1, r)), so no range crosses a tile boundary; workgroups
// p >= s * T_sk get no Stream-K work.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define GSK_HD __host__ __device__ __forceinline__
#else
#define GSK_HD inline
#endif

namespace gsk {

struct Partition {
    int32_t tiles_m, tiles_n;
    int32_t T;        // output tiles
    int32_t ipt;      // MAC iterations per tile
    int32_t T_sk;     // tiles split by Stream-K (a prefix of the tile ids)
    int32_t g;        // Stream-K workgroups
    int32_t q, r;     // T_sk * ipt = q * g + r
    int32_t grid;     // launched workgroups (also the data-parallel tile stride)
    int32_t group_m;  // tile-order group height; <= 0 means row-major order
    int32_t xcds;     // dies that hardware workgroup ids are dealt to in turn
    int32_t k_aligned; // walk a Stream-K range as whole tiles, head piece, tail
                       // piece (see work_next); only with the split fixup
    int32_t hilbert;   // tile order: 1 = Hilbert curve over the tile grid
    int32_t sk_split;  // 0: the even split of all T_sk * ipt iterations over g
                       // workgroups; s > 0: each Stream-K tile cut into s pieces
};

GSK_HD int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// First Stream-K iteration of workgroup p (p may equal g: the end of the
// last range).  Ranges are contiguous, ascending in p, and differ in length
// by at most one (issue #1393, the first-wave kernel's start/last iteration).
GSK_HD int64_t sk_begin(const Partition &P, int64_t p)
{
    if (P.sk_split > 0) {
        const int64_t t = p / P.sk_split, j = p - t * P.sk_split;
        if (t >= P.T_sk)
            return (int64_t)P.T_sk * P.ipt;
        return t * P.ipt + j * P.q + min64(j, P.r);
    }
    return p * P.q + min64(p, P.r);
}

// The workgroup whose Stream-K range holds global iteration it
// (0 <= it < T_sk * ipt): the inverse of sk_begin.
GSK_HD int32_t sk_wg_of_iter(const Partition &P, int64_t it)
{
    int64_t long_part = (int64_t)P.r * (P.q + 1);  // the r ranges of length q+1
    if (P.sk_split > 0) {
        // within tile t, the same rule over its ipt iterations (q >= 1)
        const int64_t t = it / P.ipt, k = it - t * P.ipt;
        const int64_t j = k < long_part ? k / (P.q + 1) : P.r + (k - long_part) / P.q;
        return (int32_t)(t * P.sk_split + j);
    }
    if (it < long_part)
        return (int32_t)(it / (P.q + 1));
    return (int32_t)(P.r + (it - long_part) / P.q);  // q > 0 whenever this is reached
}

// Tile (x, y) of the t-th cell of the grid [0, gm) x [0, gn) in Hilbert-curve
// order ("Inside NVIDIA GPUs: Anatomy of high performance matmul kernels"
// page: Hilbert curves as a tile scheduling policy).  The curve is the classic
// one on the power-of-two square of side >= max(gm, gn), restricted to the
// cells inside the grid: t counts in-grid cells only, so the map is a
// bijection on [0, gm * gn) for any grid, and on a power-of-two square grid
// it is the textbook curve.
//
// Top-down walk: the current square is mapped to the grid by an affine map
// x = ox + a*u + b*v, y = oy + c*u + d*v of its local (u, v) (a, b, c, d in
// {-1, 0, 1}).  Its four quadrants are visited in the curve's order
// (0,0) (0,h) (h,h) (h,0) (local, h the half side), the first transposed and
// the last anti-transposed; the walk counts each quadrant's cells inside the
// grid, enters the one holding cell t, and composes its map.
GSK_HD void hilbert_coords(int32_t gm, int32_t gn, int32_t t, int32_t *x, int32_t *y)
{
    int32_t side = 1;
    while (side < gm || side < gn)
        side *= 2;
    int32_t ox = 0, oy = 0, a = 1, b = 0, c = 0, d = 1;
    for (int32_t s = side; s > 1; s /= 2) {
        const int32_t h = s / 2;
        for (int32_t q = 0; q < 4; ++q) {
            // quadrant q: local offset (p, r) and map (u, v) = (p + e*u' + f*v', r + g*u' + k*v')
            int32_t p, r, e, f, g, k;
            if (q == 0) {
                p = 0; r = 0; e = 0; f = 1; g = 1; k = 0;
            } else if (q == 1) {
                p = 0; r = h; e = 1; f = 0; g = 0; k = 1;
            } else if (q == 2) {
                p = h; r = h; e = 1; f = 0; g = 0; k = 1;
            } else {
                p = 2 * h - 1; r = h - 1; e = 0; f = -1; g = -1; k = 0;
            }
            // the quadrant's cells in grid coordinates: the image of the
            // local cells [qu, qu + h) x [qv, qv + h) of the current square
            const int32_t qu = q >= 2 ? h : 0, qv = (q == 1 || q == 2) ? h : 0;
            const int32_t x0 = ox + a * qu + b * qv, x1 = ox + a * (qu + h - 1) + b * (qv + h - 1);
            const int32_t y0 = oy + c * qu + d * qv, y1 = oy + c * (qu + h - 1) + d * (qv + h - 1);
            const int32_t xl = x0 < x1 ? x0 : x1, xh = (x0 < x1 ? x1 : x0) + 1;
            const int32_t yl = y0 < y1 ? y0 : y1, yh = (y0 < y1 ? y1 : y0) + 1;
            const int32_t nx = (xh < gm ? xh : gm) - (xl > 0 ? xl : 0);
            const int32_t ny = (yh < gn ? yh : gn) - (yl > 0 ? yl : 0);
            const int32_t cells = nx > 0 && ny > 0 ? nx * ny : 0;
            if (t < cells || q == 3) {
                const int32_t ox2 = ox + a * p + b * r, oy2 = oy + c * p + d * r;
                const int32_t a2 = a * e + b * g, b2 = a * f + b * k;
                const int32_t c2 = c * e + d * g, d2 = c * f + d * k;
                ox = ox2; oy = oy2; a = a2; b = b2; c = c2; d = d2;
                break;
            }
            t -= cells;
        }
    }
    *x = ox;
    *y = oy;
}

// Output tile (tile_m, tile_n) of tile id t.
//  - hilbert: the Hilbert-curve order above over the tiles_m x tiles_n grid;
//  - group_m > 0: issue #1393's GROUP_M re-ordering "for better L2
//    performance" (the final revision's swizzle_tile): ids walk down a band of
//    group_m tile rows before moving one tile column right, so tiles that run
//    at the same time share A row panels and B column panels in cache; in a
//    shorter last band the row is tile_id mod (band height) of the global id,
//    as on the page;
//  - otherwise row-major.
GSK_HD void tile_coords(const Partition &P, int32_t t, int32_t *tm, int32_t *tn)
{
    if (P.hilbert) {
        hilbert_coords(P.tiles_m, P.tiles_n, t, tm, tn);
        return;
    }
    if (P.group_m <= 0) {
        *tm = t / P.tiles_n;
        *tn = t - (t / P.tiles_n) * P.tiles_n;
        return;
    }
    int32_t band = P.group_m * P.tiles_n;        // tiles per band of group_m rows
    int32_t b = t / band;
    int32_t first_row = b * P.group_m;
    int32_t rows = P.tiles_m - first_row;        // the last band may be shorter
    if (rows > P.group_m)
        rows = P.group_m;
    int32_t in_band = t - b * band;
    *tm = first_row + t % rows;
    *tn = in_band / rows;
}

// Logical workgroup run by hardware workgroup id hw.  The dispatcher deals
// consecutive hardware ids to the xcds dies in turn (id mod xcds), and each
// die has its own L2.  The remap hands die x a contiguous block of logical
// ids instead, so neighbouring tiles (which share operand panels) run on the
// same die.  It is a bijection on [0, grid).
GSK_HD int32_t logical_wg(int32_t hw, int32_t grid, int32_t xcds)
{
    if (xcds <= 1)
        return hw;
    int32_t die = hw % xcds;
    int32_t slot = hw / xcds;
    int32_t per_die = grid / xcds;
    int32_t extra = grid - per_die * xcds;       // the first `extra` dies get one more
    return die * per_die + (die < extra ? die : extra) + slot;
}

enum Role { ROLE_FULL = 0, ROLE_CONTRIB = 1, ROLE_OWNER = 2 };

struct WorkItem {
    int32_t tile;       // tile id
    int32_t kb, ke;     // MAC iterations [kb, ke) of the tile
    int32_t role;       // Role
    int32_t peer_last;  // OWNER: last workgroup holding a partial of this tile
};

struct WorkCursor {
    int64_t it, end;    // Stream-K iterations still to walk (in order mode)
    int64_t b, e;       // the workgroup's whole Stream-K range (k-aligned mode)
    int32_t full;       // next whole tile of the range (k-aligned mode)
    int32_t phase;      // k-aligned mode: 0 whole tiles, 1 head piece, 2 tail piece, 3 done
    int32_t dp_tile;    // next data-parallel tile
};

GSK_HD WorkCursor work_begin(const Partition &P, int32_t p)
{
    WorkCursor c;
    if (P.T_sk > 0 && p < P.g) {
        c.it = sk_begin(P, p);
        c.end = sk_begin(P, p + 1);
    } else {
        c.it = c.end = 0;
    }
    c.b = c.it;
    c.e = c.end;
    c.full = (int32_t)((c.b + P.ipt - 1) / (P.ipt > 0 ? P.ipt : 1));
    c.phase = 0;
    c.dp_tile = P.T_sk + p;
    return c;
}

GSK_HD void set_owner(const Partition &P, int32_t p, int32_t tile, int32_t ke, WorkItem &w)
{
    w.tile = tile;
    w.kb = 0;
    w.ke = ke;
    w.role = ROLE_OWNER;
    w.peer_last = sk_wg_of_iter(P, (int64_t)tile * P.ipt + P.ipt - 1);
    (void)p;
}

// Next unit of work of workgroup p.  The Stream-K range is cut at tile
// boundaries (issue #1393, the final revision's while loop over
// [start_iter, last_iter)); then the data-parallel tiles T_sk + p,
// T_sk + p + grid, ... follow.  Only the first Stream-K segment can start
// inside a tile (CONTRIB) and only the last can stop inside one (OWNER).
//
// k-aligned mode (with the split fixup, where every piece is parked and the
// order of a workgroup's segments does not matter): the same segments, but
// whole tiles first, then the head piece (k = 0 up), then the tail piece.
// All workgroups then start their head pieces at k = 0 together and their
// tail pieces at the same offset from their start, so the workgroups running
// side by side read the same k range of A and B at the same time, as in a
// data-parallel wave, and share it in L2.  (In order mode the tail pieces
// start at k offsets that differ from workgroup to workgroup.)
GSK_HD bool work_next(const Partition &P, int32_t p, WorkCursor &c, WorkItem &w)
{
    if (P.k_aligned) {
        const int64_t b = c.b, e = c.e;
        if (b >= e) {
            c.phase = 3;
        } else if (c.phase < 3) {
            if (c.phase == 0) {
                if (((int64_t)c.full + 1) * P.ipt <= e) {
                    w.tile = c.full;
                    w.kb = 0;
                    w.ke = P.ipt;
                    w.role = ROLE_FULL;
                    w.peer_last = p;
                    ++c.full;
                    return true;
                }
                c.phase = 1;
            }
            if (c.phase == 1) {
                c.phase = 2;
                const int32_t t = (int32_t)(e / P.ipt);
                const int32_t ke = (int32_t)(e - (int64_t)t * P.ipt);
                if (ke > 0 && (int64_t)t * P.ipt >= b) {
                    set_owner(P, p, t, ke, w);
                    return true;
                }
            }
            if (c.phase == 2) {
                c.phase = 3;
                const int32_t t = (int32_t)(b / P.ipt);
                const int32_t kb = (int32_t)(b - (int64_t)t * P.ipt);
                if (kb > 0) {
                    const int64_t tile_end = (int64_t)(t + 1) * P.ipt;
                    w.tile = t;
                    w.kb = kb;
                    w.ke = (int32_t)((e < tile_end ? e : tile_end) - (int64_t)t * P.ipt);
                    w.role = ROLE_CONTRIB;
                    w.peer_last = p;
                    return true;
                }
            }
        }
    } else if (c.it < c.end) {
        int32_t tile = (int32_t)(c.it / P.ipt);
        int32_t kb = (int32_t)(c.it - (int64_t)tile * P.ipt);
        int64_t left = c.end - c.it;
        int32_t ke = (P.ipt - kb <= left) ? P.ipt : kb + (int32_t)left;
        w.tile = tile;
        w.kb = kb;
        w.ke = ke;
        w.peer_last = p;
        if (kb != 0) {
            w.role = ROLE_CONTRIB;
        } else if (ke == P.ipt) {
            w.role = ROLE_FULL;
        } else {
            set_owner(P, p, tile, ke, w);
        }
        c.it += ke - kb;
        return true;
    }
    if (c.dp_tile < P.T) {
        w.tile = c.dp_tile;
        w.kb = 0;
        w.ke = P.ipt;
        w.role = ROLE_FULL;
        w.peer_last = p;
        c.dp_tile += P.grid;
        return true;
    }
    return false;
}

// Workgroups [*first, *last] share Stream-K tile t (t < T_sk); they are
// more than one exactly when the tile is split.
GSK_HD void tile_workers(const Partition &P, int32_t t, int32_t *first, int32_t *last)
{
    *first = sk_wg_of_iter(P, (int64_t)t * P.ipt);
    *last = sk_wg_of_iter(P, (int64_t)t * P.ipt + P.ipt - 1);
}

// Workspace slot of workgroup p's piece of a split tile: a piece that starts
// inside the tile (always the workgroup's first segment) uses slot 2p, the
// head piece (k = 0, always the workgroup's last segment) slot 2p + 1.
GSK_HD int32_t split_slot(int32_t p, bool head) { return 2 * p + (head ? 1 : 0); }

// Split tiles workgroup p took part in (at most two: the tile its range
// starts in and the tile it ends in); returns how many were written.
GSK_HD int split_tiles_of(const Partition &P, int32_t p, int32_t out[2])
{
    int n = 0;
    if (P.T_sk <= 0 || p >= P.g)
        return 0;
    const int64_t b = sk_begin(P, p), e = sk_begin(P, p + 1);
    if (b >= e)
        return 0;
    const int32_t t0 = (int32_t)(b / P.ipt), t1 = (int32_t)((e - 1) / P.ipt);
    int32_t f, l;
    tile_workers(P, t0, &f, &l);
    if (f != l)
        out[n++] = t0;
    if (t1 != t0) {
        tile_workers(P, t1, &f, &l);
        if (f != l)
            out[n++] = t1;
    }
    return n;
}

// Share of blocks [*b0, *b1) of a split tile (nblocks 32x32 blocks) reduced
// by the i-th of its n workgroups.
GSK_HD void split_share(int32_t i, int32_t n, int32_t nblocks, int32_t *b0, int32_t *b1)
{
    *b0 = (int32_t)((int64_t)i * nblocks / n);
    *b1 = (int32_t)((int64_t)(i + 1) * nblocks / n);
}

}  // namespace gsk
