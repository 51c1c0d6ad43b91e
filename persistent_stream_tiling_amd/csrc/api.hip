// Host side of the C ABI: plan creation (tile grid, schedule partition,
// workspace layout), introspection and the launch path.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <new>
#include <string>

#include "gemm_sk.h"
#include "kernels.h"
#include "schedule.h"

using namespace gsk;

struct gemm_plan {
    int64_t M, N, K;
    int dtype, schedule;
    int bm, bn, bk, group_m;
    uint32_t flags;
    const Variant *variant;
    Partition P;
    int64_t iters_sk;
    int cus, xcds, wg_capacity;
    int device;                // HIP device ordinal, -1 for a described device
    int pack_a, pack_b;
    int64_t lda, ldb;          // leading dimensions the kernel reads (packed or not)
    size_t off_flags, off_counters, off_partials, off_pack_a, off_pack_b, ws_size;
    int32_t spin_limit;
    int32_t drop_wg;           // GEMM_FLAG_DEBUG_DROP_SIGNAL: workgroup that never signals
    int split_fixup, max_pieces;
    bool grid_from_model;      // tile and g picked by the Stream-K cost model
};

namespace {

thread_local std::string g_error;

void set_error(const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
}

int elem_size(int dtype) { return dtype == GEMM_F32 ? 4 : (dtype == GEMM_I8 ? 1 : 2); }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Default output tile for fp16/bf16 when the caller names none.
//
// Tile-per-workgroup schedules (DP, persistent): a wave-quantisation model.
// A launch runs ceil(T / CUs) waves of tiles; a wave costs the tile shape's
// fixed part (launch, prologue, C stores) plus ipt MAC iterations (64 deep)
// at the per-iteration time that shape sustains.  Both are least-squares fits
// to one-tile-per-workgroup launches of 86-235 log-sampled fp16 shapes on
// MI355X (fp16 C; the sweep of the Stream-K cost model): 19.0 + 1.22 us per
// iteration at 256x256, 13.0 + 0.97 at 256x128 (128x256, not in the sweep,
// 1.3% faster per iteration as an earlier ring-kernel measurement had it),
// 12.3 + 0.78 at 128x128, 7.9 + 1.00 at 64x64 (the register-staged kernel,
// a candidate only while it gives at most one tile per CU).  The cheapest
// estimate wins; ties go to the larger tile.  Big tiles win once there are
// enough of them to fill the CUs (4096^3: 256x256), smaller ones when the big
// ones would leave CUs idle (1536x1536x8192: 128x128), and 64x64 on the
// smallest short-K shapes, where the fixed part dominates.
//
// Stream-K and hybrid spread the MAC iterations over all workgroups whatever
// the tile, so the tile decides the efficiency of the MAC loop and the size
// of the fixup: 256x256 when there are at least CUs/2 such tiles, otherwise
// 256x128 (measured faster on the wave-quantised and long-K shapes, where
// most tiles are split).
struct TileChoice {
    int bm, bn;
    double fixed_us, iter_us;
};
static const TileChoice kTileModel[] = {{256, 256, 19.0, 1.22},
                                        {256, 128, 13.0, 0.97},
                                        {128, 256, 13.0, 0.957},
                                        {128, 128, 12.3, 0.78},
                                        {64, 64, 7.9, 1.00}};

void default_tile(int64_t M, int64_t N, int64_t K, gemm_schedule schedule, int cus, int *bm,
                  int *bn)
{
    const int64_t t256 = cdiv(M, 256) * cdiv(N, 256);
    if (schedule == GEMM_STREAMK || schedule == GEMM_HYBRID) {
        *bm = 256;
        *bn = t256 * 2 >= cus ? 256 : 128;
        return;
    }
    const int64_t ipt = cdiv(K > 0 ? K : 1, 64);
    double best = 0.0;
    for (const TileChoice &c : kTileModel) {
        const int64_t T = cdiv(M, c.bm) * cdiv(N, c.bn);
        if (c.bm == 64 && T > cus)
            continue;
        const double est = (double)cdiv(T, cus) * (c.fixed_us + (double)ipt * c.iter_us);
        if (&c == kTileModel || est < best) {
            best = est;
            *bm = c.bm;
            *bn = c.bn;
        }
    }
}

// Default Stream-K / hybrid plan for fp16/bf16 when the caller names neither a
// tile nor a grid.  The Triton Stream-K issue's benchmark picks g per shape
// from a sweep; a library call cannot sweep, so the planner estimates a few
// candidate plans and takes the cheapest.  Candidates, for each of the tiles
// 256x256, 256x128, 128x128, and 64x64 where it gives at most CUs tiles, with
// T tiles of ipt 64-deep iterations:
//   - g = s*T for s in {1, 2, 3, 4, 6, 8, 16} dividing ipt, g <= CUs: every
//     workgroup runs one piece of exactly ipt/s iterations of one tile (s = 1
//     is one whole tile per workgroup, no fixup);
//   - g = CUs when that does not split the tiles evenly: Stream-K's even
//     split of all T*ipt iterations, whose ranges cross tile boundaries.
// Estimated us, with q the iterations of the longest range and a = bm*bn/65536:
//   c0 + it[tile]*q + [s > 1]*(split[tile] + c_log*a*log2(s))
//      + [ranges cross tiles]*cross
// The numbers are a least-squares fit to MI355X measurements of these
// candidates on 260 log-sampled fp16 shapes (mean data-parallel time / model
// pick 1.22 there, also in two-fold cross-validation, against 0.99 for one
// workgroup per CU); `cross` is what a
// workgroup running pieces of two tiles costs: a second pipeline fill and a
// second parked piece, which the tile's whole fixup then waits for.  Returns
// false (keep the one-workgroup-per-CU default) when every tile shape has more
// than CUs tiles.
struct StreamKModel {
    double c0, it[4], split[4], c_log, cross;
};
static const StreamKModel kSkModel = {13.31, {1.313, 0.979, 0.772, 0.929},
                                      {15.36, 9.15, 6.42, 2.35}, 0.08, 10.03};
static const int kSkTiles[4][2] = {{256, 256}, {256, 128}, {128, 128}, {64, 64}};
// 64x64 (the register-staged kernel) is a candidate only while it gives at most
// one tile per CU: slow per FLOP, it wins only where fixed per-tile costs dominate
constexpr int kSkSmallTile = 3;
static const int kSkSplits[] = {1, 2, 3, 4, 6, 8, 16};

double streamk_estimate(int ti, int64_t T, int64_t ipt, int64_t g)
{
    const StreamKModel &m = kSkModel;
    const double area = kSkTiles[ti][0] * kSkTiles[ti][1] / 65536.0;
    const bool aligned = g % T == 0 && ipt % (g / T) == 0;
    const int64_t s = aligned ? g / T : std::max<int64_t>(2, cdiv(g, T));
    const int64_t q = aligned ? ipt / s : cdiv(T * ipt, g);
    double est = m.c0 + m.it[ti] * (double)q + (aligned ? 0.0 : m.cross);
    if (s > 1)
        est += m.split[ti] + m.c_log * area * std::log2((double)s);
    return est;
}

bool streamk_default_plan(int64_t M, int64_t N, int64_t K, int cus, int *bm, int *bn, int *grid)
{
    const int64_t ipt = cdiv(K > 0 ? K : 1, 64);
    double best = 0.0;
    bool found = false, any_aligned = false;
    for (int ti = 0; ti < 4; ++ti) {
        const int64_t T = cdiv(M, kSkTiles[ti][0]) * cdiv(N, kSkTiles[ti][1]);
        if (T <= 0 || (ti == kSkSmallTile && T > cus))
            continue;
        auto consider = [&](int64_t g) {
            const double e = streamk_estimate(ti, T, ipt, g);
            if (!found || e < best) {
                best = e;
                found = true;
                *bm = kSkTiles[ti][0];
                *bn = kSkTiles[ti][1];
                *grid = (int)g;
            }
        };
        for (int s : kSkSplits)
            if (ipt % s == 0 && s * T <= cus) {
                any_aligned = true;
                consider(s * T);
            }
        const int64_t g = cus;
        if (T * ipt >= g && !(g % T == 0 && ipt % (g / T) == 0))
            consider(g);
    }
    return found && any_aligned;
}

// The first compiled variant matching the request (0 = any): the table lists
// each dtype's preferred kernel for a tile first.
const Variant *find_variant(int dtype, const gemm_tiles &t)
{
    // fp16/bf16 prefer the direct-to-LDS ring kernel and fall back to the
    // register-staged one for tiles it does not cover (64x64); int8 has the
    // ping-pong kernel (256x256) and the register-staged one; fp32 runs the
    // register-staged kernel only
    const bool staged_only = dtype == GEMM_F32;
    int n = 0;
    const Variant *v = variants(&n);
    // kinds in order of preference: the ping-pong kernel where one is built
    // (256x256), then the ring kernel, then the register-staged one;
    // GEMM_FLAG_PING_PONG asks for the first only, GEMM_FLAG_RING_KERNEL
    // skips it
    int kinds[3] = {3, 2, 0};
    if (staged_only)
        kinds[0] = 0, kinds[1] = kinds[2] = -1;
    else if (t.flags & GEMM_FLAG_PING_PONG)
        kinds[1] = kinds[2] = -1;
    else if (t.flags & GEMM_FLAG_RING_KERNEL)
        kinds[0] = 2, kinds[1] = 0, kinds[2] = -1;
    for (int ki = 0; ki < 3 && kinds[ki] >= 0; ++ki)
        for (int i = 0; i < n; ++i)
            if (v[i].dtype == dtype && v[i].bm == t.bm && v[i].bn == t.bn && v[i].kind == kinds[ki] &&
                (v[i].stream_copies != 0) == ((t.flags & GEMM_FLAG_STREAM_COPIES) != 0) &&
                (t.wave_m == 0 || v[i].wave_m == t.wave_m) &&
                (t.wave_n == 0 || v[i].wave_n == t.wave_n) && (t.bk == 0 || v[i].bk == t.bk) &&
                (t.stages == 0 || v[i].stages == t.stages))
                return &v[i];
    return nullptr;
}

// Flag bits of kernel families that are no longer built.
constexpr uint32_t kReservedFlags = (1u << 2) | (1u << 5);

// Polls before a fixup wait gives up.  A poll is a sleep of ~128 cycles plus a
// memory round trip, so this is about a second: orders of magnitude beyond a
// real wait (one workgroup's Stream-K share, milliseconds at most), and it
// turns a lost signal into an error instead of a hung GPU.
constexpr int32_t kSpinLimit = 1 << 21;
// int8: |a*b| <= 2^14, so sums over K < 2^17 stay inside int32
constexpr int64_t kI8MaxK = (int64_t)1 << 17;
// GEMM_FLAG_DEBUG_DROP_SIGNAL plans: a few milliseconds
constexpr int32_t kDebugSpinLimit = 4096;

constexpr int kDiesPerGfx950 = 8;

gemm_plan *create(int64_t M, int64_t N, int64_t K, gemm_dtype dtype, gemm_schedule schedule,
                  const gemm_tiles *tiles_in, const gemm_device_desc &dev, int device,
                  bool query_occupancy)
{
    if (M < 0 || N < 0 || K < 0) {
        set_error("negative size M=%lld N=%lld K=%lld", (long long)M, (long long)N, (long long)K);
        return nullptr;
    }
    if (dtype != GEMM_F32 && dtype != GEMM_F16 && dtype != GEMM_BF16 && dtype != GEMM_I8) {
        set_error("unknown dtype %d", (int)dtype);
        return nullptr;
    }
    if (schedule < GEMM_DP || schedule > GEMM_HYBRID) {
        set_error("unknown schedule %d", (int)schedule);
        return nullptr;
    }
    if (dev.cus < 1 || dev.xcds < 1 || dev.wg_per_cu < 0) {
        set_error("bad device description cus=%d xcds=%d wg_per_cu=%d", dev.cus, dev.xcds,
                  dev.wg_per_cu);
        return nullptr;
    }
    gemm_tiles t = {};
    if (tiles_in)
        t = *tiles_in;
    if (t.flags & kReservedFlags) {
        set_error("flags 0x%x: bits 2 and 5 are reserved", t.flags & kReservedFlags);
        return nullptr;
    }
    if ((t.flags & GEMM_FLAG_PING_PONG) && (t.flags & GEMM_FLAG_RING_KERNEL)) {
        set_error("GEMM_FLAG_PING_PONG and GEMM_FLAG_RING_KERNEL exclude each other");
        return nullptr;
    }
    const int E = elem_size(dtype);
    bool grid_from_model = false;
    // the default hybrid plan where the cost model does not apply (more tiles
    // than CUs for every tile shape): one Stream-K wave (T_sk = T mod g, as
    // with GEMM_FLAG_ONE_TILE), its tiles cut into their own pieces
    bool default_hybrid_split = false;
    if (t.bm == 0 && t.bn == 0) {
        if (dtype == GEMM_F32)
            t.bm = t.bn = (M * N <= 512 * 512) ? 64 : 128;
        else if (dtype == GEMM_I8)
            t.bm = t.bn = cdiv(M, 256) * cdiv(N, 256) >= dev.cus ? 256 : 128;
        else {
            // Stream-K / hybrid with neither a tile nor a grid (and no kernel
            // asked for): the cost model picks both
            const uint32_t kernel_flags =
                GEMM_FLAG_PING_PONG | GEMM_FLAG_RING_KERNEL | GEMM_FLAG_STREAM_COPIES;
            const bool default_plan = (schedule == GEMM_STREAMK || schedule == GEMM_HYBRID) &&
                                      t.grid == 0 && t.bk == 0 && t.wave_m == 0 &&
                                      t.wave_n == 0 && t.stages == 0 && !(t.flags & kernel_flags);
            int bm = 0, bn = 0, grid = 0;
            if (default_plan && streamk_default_plan(M, N, K, dev.cus, &bm, &bn, &grid)) {
                t.bm = bm, t.bn = bn, t.grid = grid;
                grid_from_model = true;
            } else {
                default_hybrid_split = default_plan && schedule == GEMM_HYBRID;
                default_tile(M, N, K, schedule, dev.cus, &t.bm, &t.bn);
                // a wave layout, ring depth or kernel family asked for may
                // exist only at the 256x256 tile
                if (!find_variant(dtype, t))
                    t.bm = t.bn = 256;
            }
        }
    } else if (t.bm == 0 || t.bn == 0) {
        set_error("give both bm and bn, or neither");
        return nullptr;
    }
    if (dtype == GEMM_I8 && K >= kI8MaxK) {
        set_error("int8: K = %lld could overflow the int32 sums (K < %lld)", (long long)K,
                  (long long)kI8MaxK);
        return nullptr;
    }
    if (dtype == GEMM_I8 && (t.flags & GEMM_FLAG_C_INPUT_DTYPE)) {
        set_error("int8 products are written as int32; GEMM_FLAG_C_INPUT_DTYPE does not apply");
        return nullptr;
    }
    const Variant *var = find_variant(dtype, t);
    if (!var) {
        set_error("no kernel for dtype %d with tile %dx%d, bk %d, waves %dx%d, stages %d, "
                  "flags 0x%x",
                  (int)dtype, t.bm, t.bn, t.bk, t.wave_m, t.wave_n, t.stages, t.flags);
        return nullptr;
    }
    if (t.grid < 0) {
        set_error("grid must be >= 0");
        return nullptr;
    }
    const int V = 16 / E;
    const int64_t lda = (K * E) % 16 ? cdiv(K, V) * V : K;
    const int64_t ldb = (N * E) % 16 ? cdiv(N, V) * V : N;
    // 32-bit index limits of the kernel: sizes, and the buffer offsets within
    // one tile's rows of A and C and one iteration's rows of B (the kernels
    // address those through a descriptor based at the tile or slab, with
    // 32-bit offsets, 0x80000000 meaning "out of range")
    const int CE = dtype == GEMM_I8 ? 4 : ((t.flags & GEMM_FLAG_C_INPUT_DTYPE) ? E : 4);
    const int64_t lim = (int64_t)1 << 30;
    if (M >= lim || N >= lim || K >= lim || (int64_t)var->bm * lda * E >= lim ||
        (int64_t)var->bk * ldb * E >= lim || (int64_t)var->bm * N * CE >= lim) {
        set_error("matrix too large for 32-bit indexing (M, N, K < 2^30 and %d rows of A, %d "
                  "rows of B and %d rows of C each below 2^30 bytes)",
                  var->bm, var->bk, var->bm);
        return nullptr;
    }

    gemm_plan *p = new (std::nothrow) gemm_plan();
    if (!p) {
        set_error("out of host memory");
        return nullptr;
    }
    p->M = M;
    p->N = N;
    p->K = K;
    p->dtype = dtype;
    p->schedule = schedule;
    p->bm = var->bm;
    p->bn = var->bn;
    p->bk = var->bk;
    p->group_m = t.group_m == 0 ? 8 : (t.group_m < 0 ? 0 : t.group_m);
    p->flags = t.flags;
    p->variant = var;
    p->cus = dev.cus;
    p->xcds = (t.flags & GEMM_FLAG_NO_XCD_REMAP) ? 1 : dev.xcds;
    p->device = device;
    p->spin_limit = kSpinLimit;
    p->drop_wg = -1;
    p->grid_from_model = grid_from_model;

    int occ = dev.wg_per_cu > 0 ? dev.wg_per_cu : 1;
    if (query_occupancy) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, var->kernel, var->threads, 0) ==
                hipSuccess &&
            n > 0)
            occ = n;
    }
    p->wg_capacity = dev.cus * occ;

    Partition &P = p->P;
    P.tiles_m = (int32_t)cdiv(M, var->bm);
    P.tiles_n = (int32_t)cdiv(N, var->bn);
    const int64_t T = (int64_t)P.tiles_m * P.tiles_n;
    const int64_t ipt = cdiv(K, var->bk);
    if (T >= lim || T * ipt >= ((int64_t)1 << 31)) {
        set_error("too many tiles or MAC iterations for 32-bit indexing");
        delete p;
        return nullptr;
    }
    P.T = (int32_t)T;
    P.ipt = (int32_t)ipt;
    P.group_m = p->group_m;
    P.hilbert = (t.flags & GEMM_FLAG_HILBERT_ORDER) ? 1 : 0;
    P.xcds = p->xcds;
    const int32_t g = t.grid > 0 ? t.grid : dev.cus;
    int64_t T_sk = 0;
    switch (schedule) {
    case GEMM_DP:
        P.g = 0;
        P.grid = (int32_t)T;
        break;
    case GEMM_PERSISTENT:
        P.g = g;
        P.grid = (int32_t)(T < g ? T : g);
        break;
    case GEMM_STREAMK:
        T_sk = T;
        P.g = g;
        P.grid = g;
        break;
    case GEMM_HYBRID:
        // Issue #1393, final revision: the last (partial) wave goes to Stream-K,
        // plus one more full wave when two_tiles is on and more than g tiles
        // would stay data-parallel.
        T_sk = T % g;
        // (the default plan above the cost model's range keeps one wave: its
        // Stream-K tiles are then fewer than g and cut per tile, below)
        if (!(t.flags & GEMM_FLAG_ONE_TILE) && !default_hybrid_split && T - T_sk > g)
            T_sk += g;
        P.g = g;
        P.grid = T_sk > 0 ? g : (int32_t)(T < g ? T : g);
        break;
    }
    if (ipt == 0 || T == 0)
        T_sk = 0;  // nothing to split: K = 0 is a fill, an empty C is a no-op
    P.T_sk = (int32_t)T_sk;
    p->iters_sk = T_sk * ipt;
    if (T_sk > 0 && ((t.flags & GEMM_FLAG_TILE_SPLIT) || (default_hybrid_split && T_sk <= g))) {
        // each Stream-K tile cut into s pieces, one per workgroup
        if (g < T_sk) {
            set_error("GEMM_FLAG_TILE_SPLIT needs g >= the %lld Stream-K tiles (g = %d)",
                      (long long)T_sk, g);
            delete p;
            return nullptr;
        }
        const int64_t s = std::min<int64_t>(g / T_sk, ipt);
        P.sk_split = (int32_t)s;
        P.q = (int32_t)(ipt / s);
        P.r = (int32_t)(ipt % s);
    } else if (T_sk > 0) {
        P.q = (int32_t)(p->iters_sk / g);
        P.r = (int32_t)(p->iters_sk % g);
    }
    if (T_sk > 0) {
        // the in-kernel fixups wait on other workgroups, which must all be
        // running; the two-kernel fixup never waits
        if (g > p->wg_capacity && !(t.flags & GEMM_FLAG_FIXUP_TWO_KERNEL)) {
            set_error("Stream-K grid %d exceeds the %d workgroups that can be resident at once; "
                      "the in-kernel fixup needs them all running together "
                      "(GEMM_FLAG_FIXUP_TWO_KERNEL has no such limit)",
                      g, p->wg_capacity);
            delete p;
            return nullptr;
        }
        // Fixup mode: split (with the k-aligned walk) whenever some tile is cut;
        // head mode only when asked for.
        p->max_pieces = 1;
        for (int32_t t = 0; t < P.T_sk; ++t) {
            int32_t f, l;
            tile_workers(P, t, &f, &l);
            if (l - f + 1 > p->max_pieces)
                p->max_pieces = l - f + 1;
        }
        if (t.flags & GEMM_FLAG_FIXUP_TWO_KERNEL)
            p->split_fixup = p->max_pieces >= 2 ? 2 : 0;
        else if (t.flags & GEMM_FLAG_FIXUP_SPLIT)
            p->split_fixup = 1;
        else if (t.flags & GEMM_FLAG_FIXUP_HEAD)
            p->split_fixup = 0;
        else
            p->split_fixup = p->max_pieces >= 2;
        P.k_aligned = p->split_fixup;
        if ((t.flags & GEMM_FLAG_DEBUG_DROP_SIGNAL) && p->split_fixup == 2) {
            set_error("GEMM_FLAG_DEBUG_DROP_SIGNAL: the two-kernel fixup has no signals");
            delete p;
            return nullptr;
        }
        if (t.flags & GEMM_FLAG_DEBUG_DROP_SIGNAL) {
            // the last workgroup whose work includes a parked piece
            for (int32_t wg = 0; wg < g; ++wg) {
                WorkCursor c = work_begin(P, wg);
                WorkItem w;
                while (work_next(P, wg, c, w))
                    if (w.role == ROLE_CONTRIB || (w.role == ROLE_OWNER && p->split_fixup))
                        p->drop_wg = wg;
            }
            p->spin_limit = kDebugSpinLimit;
        }
        const int64_t slots = p->split_fixup ? 2 * (int64_t)g : g;
        if (slots * var->bm * var->bn * 4 >= ((int64_t)1 << 31)) {
            set_error("Stream-K grid %d too large for the partial-tile workspace indexing", g);
            delete p;
            return nullptr;
        }
    } else {
        P.q = P.r = 0;
        p->max_pieces = 1;
        p->split_fixup = 0;
        P.k_aligned = 0;
    }
    if ((t.flags & GEMM_FLAG_DEBUG_DROP_SIGNAL) && p->drop_wg < 0) {
        set_error("GEMM_FLAG_DEBUG_DROP_SIGNAL needs a plan that splits some tile");
        delete p;
        return nullptr;
    }

    // Workspace: [status word | flags | per-tile counters (split fixup) |
    //             partial tiles | packed A | packed B]; head fixup: one flag and
    //             slot per workgroup, split fixup: two of each.
    p->pack_a = lda != K && M > 0 && K > 0;
    p->pack_b = ldb != N && N > 0 && K > 0;
    p->lda = lda;
    p->ldb = ldb;
    size_t off = 0;
    if (T_sk > 0) {
        const size_t slots = p->split_fixup ? 2 * (size_t)g : (size_t)g;
        off = 256;
        p->off_flags = off;
        off = align_up(off + sizeof(int32_t) * slots, 256);
        p->off_counters = off;
        if (p->split_fixup)
            off = align_up(off + sizeof(int32_t) * (size_t)T_sk, 256);
        p->off_partials = off;
        off += sizeof(float) * slots * var->bm * var->bn;
    }
    if (p->pack_a) {
        off = align_up(off, 256);
        p->off_pack_a = off;
        off += (size_t)M * lda * E;
    }
    if (p->pack_b) {
        off = align_up(off, 256);
        p->off_pack_b = off;
        off += (size_t)K * ldb * E;
    }
    p->ws_size = off ? align_up(off, 256) : 0;
    return p;
}

const char *sched_name(int s)
{
    static const char *names[] = {"dp", "persistent", "streamk", "hybrid"};
    return (s >= 0 && s < 4) ? names[s] : "?";
}

const char *dtype_name(int d)
{
    static const char *names[] = {"f32", "f16", "bf16", "i8"};
    return (d >= 0 && d < 4) ? names[d] : "?";
}

}  // namespace

extern "C" {

gemm_plan *gemm_plan_create(int64_t M, int64_t N, int64_t K, gemm_dtype dtype,
                            gemm_schedule schedule, const gemm_tiles *tiles)
{
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) {
        set_error("no HIP device");
        return nullptr;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) !=
            hipSuccess ||
        cus < 1) {
        set_error("cannot query the compute-unit count of device %d", device);
        return nullptr;
    }
    gemm_device_desc dev = {cus, kDiesPerGfx950, 0};
    return create(M, N, K, dtype, schedule, tiles, dev, device, true);
}

gemm_plan *gemm_plan_create_for_device(int64_t M, int64_t N, int64_t K, gemm_dtype dtype,
                                       gemm_schedule schedule, const gemm_tiles *tiles,
                                       const gemm_device_desc *device)
{
    if (!device) {
        set_error("device description is NULL");
        return nullptr;
    }
    return create(M, N, K, dtype, schedule, tiles, *device, -1, false);
}

void gemm_plan_destroy(gemm_plan *plan) { delete plan; }

size_t gemm_plan_workspace_size(const gemm_plan *plan) { return plan ? plan->ws_size : 0; }

const char *gemm_last_error(void) { return g_error.c_str(); }

int gemm_plan_get_info(const gemm_plan *p, gemm_plan_info *o)
{
    if (!p || !o) {
        set_error("NULL argument");
        return -1;
    }
    memset(o, 0, sizeof *o);
    o->M = p->M;
    o->N = p->N;
    o->K = p->K;
    o->dtype = p->dtype;
    o->schedule = p->schedule;
    o->bm = p->bm;
    o->bn = p->bn;
    o->bk = p->bk;
    o->group_m = p->group_m;
    o->flags = p->flags;
    o->wave_m = p->variant->wave_m;
    o->wave_n = p->variant->wave_n;
    o->kernel_kind = p->variant->kind;
    o->stages = p->variant->stages;
    o->split_fixup = p->split_fixup;
    o->max_pieces = p->max_pieces;
    o->tiles_m = p->P.tiles_m;
    o->tiles_n = p->P.tiles_n;
    o->tiles = p->P.T;
    o->iters_per_tile = p->P.ipt;
    o->tiles_sk = p->P.T_sk;
    o->tiles_dp = p->P.T - p->P.T_sk;
    o->iters_sk = p->iters_sk;
    o->q = p->P.q;
    o->r = p->P.r;
    o->g = p->P.g;
    o->launch_grid = p->P.grid;
    o->threads = p->variant->threads;
    o->cus = p->cus;
    o->xcds = p->xcds;
    o->wg_capacity = p->wg_capacity;
    o->pack_a = p->pack_a;
    o->pack_b = p->pack_b;
    o->workspace = p->ws_size;
    o->lds_bytes = p->variant->lds_bytes;
    o->pieces_per_tile = p->P.sk_split;
    return 0;
}

int gemm_plan_describe(const gemm_plan *p, char *buf, size_t len)
{
    if (!p) {
        set_error("NULL plan");
        return -1;
    }
    char split[48] = "";
    if (p->P.sk_split > 0)
        snprintf(split, sizeof split, " tile-split x%d", p->P.sk_split);
    char order[32];
    if (p->P.hilbert)
        snprintf(order, sizeof order, "hilbert");
    else if (p->group_m > 0)
        snprintf(order, sizeof order, "bands%d", p->group_m);
    else
        snprintf(order, sizeof order, "rows");
    return snprintf(buf, buf ? len : 0,
                    "M,N,K=%lld,%lld,%lld %s C=%s %s tile=%dx%dx%d waves=%dx%d %s%d order=%s | tiles %dx%d=%d "
                    "ipt=%d | T_sk=%d T_dp=%d I_sk=%lld g=%d%s%s q=%d r=%d | grid=%d x %d threads, "
                    "lds=%zu B, capacity=%d wg, xcds=%d | fixup=%s pieces<=%d | pack A=%d B=%d | "
                    "workspace=%zu B",
                    (long long)p->M, (long long)p->N, (long long)p->K, dtype_name(p->dtype),
                    p->dtype == GEMM_I8 ? "i32"
                                        : dtype_name((p->flags & GEMM_FLAG_C_INPUT_DTYPE)
                                                         ? p->dtype
                                                         : GEMM_F32),
                    sched_name(p->schedule), p->bm, p->bn, p->bk, p->variant->wave_m,
                    p->variant->wave_n, p->variant->kind == 3 ? "pingpong" : p->variant->kind == 2 ? "ring" : "staged",
                    p->variant->kind ? p->variant->stages : 2,
                    order, p->P.tiles_m,
                    p->P.tiles_n, p->P.T, p->P.ipt, p->P.T_sk, p->P.T - p->P.T_sk,
                    (long long)p->iters_sk, p->P.g, p->grid_from_model ? " (cost model)" : "", split,
                    p->P.q, p->P.r, p->P.grid,
                    p->variant->threads, p->variant->lds_bytes, p->wg_capacity, p->xcds,
                    p->P.T_sk == 0 ? "none"
                                   : (p->split_fixup == 2 ? "two-kernel"
                                                          : (p->split_fixup ? "split" : "head")),
                    p->max_pieces, p->pack_a, p->pack_b, p->ws_size);
}

int gemm_plan_segments(const gemm_plan *p, int32_t wg, gemm_segment *out, int32_t max)
{
    if (!p || wg < 0 || wg >= (p->P.grid > 0 ? p->P.grid : 1) || (max > 0 && !out)) {
        set_error("bad argument");
        return -1;
    }
    if (p->P.T == 0 || p->P.ipt == 0)
        return 0;
    WorkCursor c = work_begin(p->P, wg);
    WorkItem w;
    int n = 0;
    while (work_next(p->P, wg, c, w)) {
        if (n < max)
            out[n] = gemm_segment{w.tile, w.kb, w.ke, w.role, w.peer_last};
        ++n;
    }
    return n;
}

int gemm_plan_tile_coords(const gemm_plan *p, int32_t t, int32_t *tm, int32_t *tn)
{
    if (!p || t < 0 || t >= p->P.T || !tm || !tn) {
        set_error("bad argument");
        return -1;
    }
    tile_coords(p->P, t, tm, tn);
    return 0;
}

int32_t gemm_plan_logical_wg(const gemm_plan *p, int32_t hw)
{
    if (!p || hw < 0 || hw >= p->P.grid) {
        set_error("bad argument");
        return -1;
    }
    return logical_wg(hw, p->P.grid, p->P.xcds);
}

int gemm_run(const gemm_plan *p, const void *A, const void *B, void *C, void *workspace,
             void *stream_v)
{
    if (!p) {
        set_error("NULL plan");
        return -1;
    }
    hipStream_t stream = (hipStream_t)stream_v;
    if (p->M == 0 || p->N == 0)
        return 0;
    if (!C) {
        set_error("C is NULL");
        return -1;
    }
    if (p->device < 0) {
        set_error("plan was made for a described device; create it with gemm_plan_create");
        return -5;
    }
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != p->device) {
        set_error("plan was made for device %d, current device is %d", p->device, cur);
        return -5;
    }
    // C holds fp32, or the input dtype with GEMM_FLAG_C_INPUT_DTYPE
    const int c_dtype = (p->flags & GEMM_FLAG_C_INPUT_DTYPE) ? p->dtype : GEMM_F32;
    const int CE = elem_size(c_dtype);
    if ((uintptr_t)C & (CE - 1)) {
        set_error("C must be %d-byte aligned", CE);
        return -1;
    }
    if (p->K == 0) {
        if (launch_zero(C, p->M * p->N, CE, stream)) {
            set_error("zero-fill launch failed: %s", hipGetErrorString(hipGetLastError()));
            return -3;
        }
        return 0;
    }
    if (!A || !B) {
        set_error("A or B is NULL");
        return -1;
    }
    if (p->ws_size && !workspace) {
        set_error("this plan needs %zu bytes of workspace", p->ws_size);
        return -2;
    }
    if (((uintptr_t)A & 15) || ((uintptr_t)B & 15) || ((uintptr_t)workspace & 255)) {
        set_error("A and B must be 16-byte aligned, workspace 256-byte aligned");
        return -1;
    }
    const int E = elem_size(p->dtype);
    uint8_t *ws = (uint8_t *)workspace;
    const uint8_t *a = (const uint8_t *)A;
    const uint8_t *b = (const uint8_t *)B;
    if (p->pack_a || p->pack_b) {
        if (launch_pack_pair(A, ws + p->off_pack_a, p->pack_a ? p->M : 0, p->K, p->K, p->lda, B,
                             ws + p->off_pack_b, p->pack_b ? p->K : 0, p->N, p->N, p->ldb, E,
                             stream)) {
            set_error("pack launch failed");
            return -3;
        }
        if (p->pack_a)
            a = ws + p->off_pack_a;
        if (p->pack_b)
            b = ws + p->off_pack_b;
    }
    KernelArgs args;
    args.A = a;
    args.B = b;
    args.C = (uint8_t *)C;
    args.c_dtype = c_dtype;
    args.status = p->P.T_sk > 0 ? (int32_t *)ws : nullptr;
    args.flags = p->P.T_sk > 0 ? (int32_t *)(ws + p->off_flags) : nullptr;
    args.partials = p->P.T_sk > 0 ? (float *)(ws + p->off_partials) : nullptr;
    args.counters = p->P.T_sk > 0 ? (int32_t *)(ws + p->off_counters) : nullptr;
    args.split_fixup = p->split_fixup;
    args.M = (int32_t)p->M;
    args.N = (int32_t)p->N;
    args.K = (int32_t)p->K;
    args.lda = (int32_t)p->lda;
    args.ldb = (int32_t)p->ldb;
    args.ldc = (int32_t)p->N;
    // a lane stores 4 consecutive elements of a row: one 16-byte (fp32) or
    // 8-byte (fp16/bf16) store when rows and C keep that alignment
    args.c_vec = (p->N % 4 == 0) && (((uintptr_t)C & (4 * CE - 1)) == 0);
    args.spin_limit = p->spin_limit;
    args.drop_signal_wg = p->drop_wg;
    args.P = p->P;
    if (p->variant->launch(args, p->P.grid, stream)) {
        set_error("kernel launch failed: %s", hipGetErrorString(hipGetLastError()));
        return -3;
    }
    // two-kernel fixup: the split tiles are reduced after every piece is parked
    if (p->split_fixup == 2 && p->variant->launch_fixup(args, p->P.T_sk, stream)) {
        set_error("fixup launch failed: %s", hipGetErrorString(hipGetLastError()));
        return -3;
    }
    return 0;
}

int32_t gemm_variant_count(void)
{
    int n = 0;
    variants(&n);
    return n;
}

int gemm_variant_get(int32_t i, gemm_variant_info *out)
{
    int n = 0;
    const Variant *v = variants(&n);
    if (!out || i < 0 || i >= n) {
        set_error("bad argument");
        return -1;
    }
    const Variant &x = v[i];
    *out = gemm_variant_info{x.dtype, x.bm,   x.bn,      x.bk,           x.wave_m, x.wave_n,
                             x.kind,  x.stages, x.stream_copies, x.threads, x.lds_bytes};
    return 0;
}

}  // extern "C"

namespace {

// Workspace of gemm_run_noalloc: one array per device, in the library's own
// device memory, held until the process ends.  In host code `scratch` is only
// a stand-in for the symbol; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is ever handed
// to a kernel or a fill.
constexpr size_t kNoAllocBytes = GEMM_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device dev, which must be current; looked up
// on the first call for that device.
void *scratch_on(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("device %d out of range for the no-alloc workspace", dev);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            set_error("no-alloc workspace: hipGetSymbolAddress failed on device %d: %s", dev,
                      hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int gemm_run_noalloc(const gemm_plan *p, const void *A, const void *B, void *C, void *stream_v)
{
    if (!p) {
        set_error("NULL plan");
        return -1;
    }
    if (p->ws_size > kNoAllocBytes) {
        set_error("plan needs %zu bytes of workspace; gemm_run_noalloc has %zu (use gemm_run "
                  "with a caller-owned workspace)",
                  p->ws_size, kNoAllocBytes);
        return -2;
    }
    if (p->ws_size == 0)
        return gemm_run(p, A, B, C, nullptr, stream_v);
    if (p->device < 0) {
        set_error("plan was made for a described device; create it with gemm_plan_create");
        return -5;
    }
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != p->device) {
        set_error("plan was made for device %d, current device is %d", p->device, cur);
        return -5;
    }
    uint8_t *ws = (uint8_t *)scratch_on(cur);
    if (!ws)
        return -3;
    // The array keeps whatever the last call on this device left: clear the
    // status word, flags and counters this plan reads (a fill kernel, not a
    // memset, so the call can be captured in a graph).  Partial slots are
    // written before they are read; repacked operands are rewritten.
    if (p->P.T_sk > 0 && p->M > 0 && p->N > 0 && p->K > 0 &&
        launch_zero(ws, (int64_t)(p->off_partials / sizeof(uint32_t)), (int)sizeof(uint32_t),
                    (hipStream_t)stream_v)) {
        set_error("workspace clear failed: %s", hipGetErrorString(hipGetLastError()));
        return -3;
    }
    return gemm_run(p, A, B, C, ws, stream_v);
}

int gemm_workspace_status(const gemm_plan *p, const void *workspace, void *stream,
                          int32_t *status)
{
    if (!p || !status) {
        set_error("NULL argument");
        return -1;
    }
    *status = 0;
    if (p->P.T_sk == 0)
        return 0;
    if (!workspace) {
        // the array gemm_run_noalloc runs in, on the current device
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess || !(workspace = scratch_on(cur)))
            return -2;
    }
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(status, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess) {
        set_error("status read failed: %s", hipGetErrorString(hipGetLastError()));
        return -3;
    }
    return 0;
}

}  // extern "C"
