// Host-thread model of the Stream-K fixup protocol (test infrastructure).
//
// One std::thread per workgroup walks its work with the library's own
// schedule code (schedule.h: work_begin / work_next / tile_workers /
// split_tiles_of / split_share), multiplies each segment in fp32 in ascending
// k, and finishes it with the workspace protocol of the gfx950 kernels:
//   - a piece of a split tile is parked in its slot, then its flag is raised
//     (release); head fixup: only pieces that do not start at k = 0, and the
//     k = 0 workgroup waits for the later ones (acquire), clears their flags
//     and adds them in ascending workgroup (= ascending k) order; split
//     fixup: every piece, and after its own MAC work each workgroup of a tile
//     waits for all of the tile's flags and reduces its share of the tile's
//     rows, head piece first then ascending k; the last reader (a counter)
//     clears the tile's flags and counter;
//   - every wait is bounded: a wait that gives up sets the status word.
// Threads start after seeded random delays and sleep at random between
// steps, so the interleavings differ from seed to seed; the result must not.
// A "drop" workgroup never raises its flag (forced failure of a signal).
// split = 2 models the two-kernel fixup: every piece is parked without a
// flag, and after all workgroups have finished (the kernel boundary) the
// split tiles are reduced in ascending k order.
//
// Usage: fixup_emulator IN OUT.  IN holds 24 int32 (see Header) then A (M*K
// fp32, row-major) and B (K*N fp32, row-major); OUT receives the status word
// (int32) and C (M*N fp32).
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "schedule.h"

using namespace gsk;

struct Header {
    int32_t M, N, K, bm, bn, bk;
    int32_t tiles_m, tiles_n, T, ipt, T_sk, g, q, r, grid, group_m, xcds, k_aligned;
    int32_t split, drop, spin_limit, seed, jitter_us, sk_split;
};

struct Shared {
    Header h;
    Partition P;
    std::vector<float> A, B, C, partials;
    std::vector<std::atomic<int32_t>> flags, counters;
    std::atomic<int32_t> status{0};
    Shared(const Header &hh, size_t slots, size_t tiles)
        : h(hh), flags(slots), counters(tiles)
    {
        for (auto &f : flags)
            f.store(0);
        for (auto &c : counters)
            c.store(0);
    }
};

static void nap(std::mt19937 &rng, int max_us)
{
    if (max_us > 0)
        std::this_thread::sleep_for(std::chrono::microseconds(rng() % (unsigned)max_us));
}

// Bounded wait for flag slot s; consumes (clears) it when asked.
static void wait_flag(Shared &S, int32_t s, bool clear)
{
    for (int32_t spins = 0; S.flags[s].load(std::memory_order_acquire) == 0; ++spins) {
        if (spins > S.h.spin_limit) {
            S.status.store(1, std::memory_order_relaxed);
            break;
        }
        std::this_thread::sleep_for(std::chrono::microseconds(5));
    }
    if (clear)
        S.flags[s].store(0, std::memory_order_relaxed);
}

static void store_c(Shared &S, const float *acc, int m0, int n0, int r0, int r1)
{
    const Header &h = S.h;
    for (int i = r0; i < r1; ++i)
        for (int j = 0; j < h.bn; ++j)
            if (m0 + i < h.M && n0 + j < h.N)
                S.C[(size_t)(m0 + i) * h.N + n0 + j] = acc[(size_t)i * h.bn + j];
}

static void workgroup(Shared &S, int32_t p)
{
    const Header &h = S.h;
    const Partition &P = S.P;
    const size_t tile_elems = (size_t)h.bm * h.bn;
    std::mt19937 rng((uint32_t)(h.seed * 1000003u + (uint32_t)p));
    nap(rng, h.jitter_us);
    std::vector<float> acc(tile_elems);
    WorkCursor c = work_begin(P, p);
    WorkItem w;
    while (work_next(P, p, c, w)) {
        int32_t tm, tn;
        tile_coords(P, w.tile, &tm, &tn);
        const int m0 = tm * h.bm, n0 = tn * h.bn;
        const int k0 = w.kb * h.bk, k1 = w.ke * h.bk < h.K ? w.ke * h.bk : h.K;
        for (int i = 0; i < h.bm; ++i)
            for (int j = 0; j < h.bn; ++j) {
                float s = 0.0f;
                if (m0 + i < h.M && n0 + j < h.N)
                    for (int k = k0; k < k1; ++k)
                        s += S.A[(size_t)(m0 + i) * h.K + k] * S.B[(size_t)k * h.N + n0 + j];
                acc[(size_t)i * h.bn + j] = s;
            }
        nap(rng, h.jitter_us);
        if (w.role == ROLE_CONTRIB || (w.role == ROLE_OWNER && h.split)) {
            const int32_t slot = h.split ? split_slot(p, w.role == ROLE_OWNER) : p;
            std::memcpy(&S.partials[(size_t)slot * tile_elems], acc.data(),
                        tile_elems * sizeof(float));
            if (p != h.drop && h.split != 2)
                S.flags[slot].store(1, std::memory_order_release);
            continue;
        }
        if (w.role == ROLE_OWNER) {
            for (int32_t q = p + 1; q <= w.peer_last; ++q)
                wait_flag(S, q, true);
            for (int32_t q = p + 1; q <= w.peer_last; ++q)
                for (size_t e = 0; e < tile_elems; ++e)
                    acc[e] += S.partials[(size_t)q * tile_elems + e];
        }
        store_c(S, acc.data(), m0, n0, 0, h.bm);
    }
    if (h.split != 1)
        return;
    int32_t tiles[2];
    const int nt = split_tiles_of(P, p, tiles);
    for (int it = 0; it < nt; ++it) {
        const int32_t t = tiles[it];
        int32_t pf, pl;
        tile_workers(P, t, &pf, &pl);
        const int32_t parts = pl - pf + 1;
        for (int32_t q = pf; q <= pl; ++q)
            wait_flag(S, split_slot(q, q == pf), false);
        int32_t r0, r1;
        split_share(p - pf, parts, h.bm, &r0, &r1);
        int32_t tm, tn;
        tile_coords(P, t, &tm, &tn);
        for (int32_t q = pf; q <= pl; ++q) {
            const float *piece = &S.partials[(size_t)split_slot(q, q == pf) * tile_elems];
            for (int i = r0; i < r1; ++i)
                for (int j = 0; j < h.bn; ++j) {
                    const size_t e = (size_t)i * h.bn + j;
                    acc[e] = q == pf ? piece[e] : acc[e] + piece[e];
                }
        }
        store_c(S, acc.data(), tm * h.bm, tn * h.bn, r0, r1);
        nap(rng, h.jitter_us);
        if (S.counters[t].fetch_add(1, std::memory_order_acq_rel) == parts - 1) {
            for (int32_t q = pf; q <= pl; ++q)
                S.flags[split_slot(q, q == pf)].store(0, std::memory_order_relaxed);
            S.counters[t].store(0, std::memory_order_relaxed);
        }
    }
}

int main(int argc, char **argv)
{
    if (argc != 3) {
        std::fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
        return 2;
    }
    FILE *f = std::fopen(argv[1], "rb");
    if (!f)
        return 2;
    Header h;
    if (std::fread(&h, sizeof h, 1, f) != 1)
        return 2;
    Partition P = {};
    P.tiles_m = h.tiles_m;
    P.tiles_n = h.tiles_n;
    P.T = h.T;
    P.ipt = h.ipt;
    P.T_sk = h.T_sk;
    P.g = h.g;
    P.q = h.q;
    P.r = h.r;
    P.grid = h.grid;
    P.group_m = h.group_m;
    P.xcds = h.xcds;
    P.k_aligned = h.k_aligned;
    P.sk_split = h.sk_split;
    const size_t slots = h.split ? 2 * (size_t)h.g : (size_t)h.g;
    Shared S(h, slots, (size_t)(h.T_sk > 0 ? h.T_sk : 1));
    S.P = P;
    S.A.resize((size_t)h.M * h.K);
    S.B.resize((size_t)h.K * h.N);
    S.C.assign((size_t)h.M * h.N, 0.0f);
    S.partials.assign(slots * (size_t)h.bm * h.bn, 0.0f);
    if (std::fread(S.A.data(), sizeof(float), S.A.size(), f) != S.A.size() ||
        std::fread(S.B.data(), sizeof(float), S.B.size(), f) != S.B.size())
        return 2;
    std::fclose(f);
    std::vector<std::thread> th;
    for (int32_t p = 0; p < h.grid; ++p)
        th.emplace_back(workgroup, std::ref(S), p);
    for (auto &t : th)
        t.join();
    if (h.split == 2) {
        // second kernel: every split tile, all rows, pieces in ascending k
        const size_t tile_elems = (size_t)h.bm * h.bn;
        std::vector<float> acc(tile_elems);
        for (int32_t t = 0; t < P.T_sk; ++t) {
            int32_t pf, pl, tm, tn;
            tile_workers(P, t, &pf, &pl);
            if (pf == pl)
                continue;
            for (int32_t q = pf; q <= pl; ++q) {
                const float *piece = &S.partials[(size_t)split_slot(q, q == pf) * tile_elems];
                for (size_t e = 0; e < tile_elems; ++e)
                    acc[e] = q == pf ? piece[e] : acc[e] + piece[e];
            }
            tile_coords(P, t, &tm, &tn);
            store_c(S, acc.data(), tm * h.bm, tn * h.bn, 0, h.bm);
        }
    }
    // a clean run leaves every flag and counter zero for the next one
    int32_t status = S.status.load();
    if (status == 0) {
        for (auto &fl : S.flags)
            if (fl.load() != 0)
                status = 2;
        for (auto &ct : S.counters)
            if (ct.load() != 0)
                status = 2;
    }
    FILE *o = std::fopen(argv[2], "wb");
    if (!o)
        return 2;
    std::fwrite(&status, sizeof status, 1, o);
    std::fwrite(S.C.data(), sizeof(float), S.C.size(), o);
    std::fclose(o);
    return 0;
}
