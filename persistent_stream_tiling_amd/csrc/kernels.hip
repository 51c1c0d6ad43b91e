// gfx950 (CDNA4) GEMM kernels: C = A.B with fp32 accumulation.  Every kernel
// runs every schedule (data-parallel, persistent, Stream-K, hybrid) in one
// launch: a workgroup walks the work items the schedule gives it (schedule.h)
// and finishes each with a store to C or a Stream-K fixup.
//
//   gemm_kernel_pair  fp16/bf16 default: 64-deep MAC iterations, operands
//                     copied straight from global memory into LDS (A in whole
//                     128-byte rows), an unrolled ring of B stages and A slots.
//   gemm_kernel       fp32, int8, and fp16/bf16 at 64x64 tiles: loads go
//                     global -> registers -> LDS, two LDS buffers.
//
// int8 inputs accumulate exactly in int32 (the pages' kernel picks an int32
// accumulator for int8); the int32 accumulators travel in the same 32-bit
// registers, partial slots and C stores as fp32 ones, and only the Stream-K
// fixup's additions differ (integer adds).
//
// All use the 32x32 MFMA with the operands swapped (B^T as the "A" operand),
// so the accumulator block holds C^T: each lane then owns four consecutive
// columns of one row of C and the epilogue writes 16-byte stores.
//
// Out-of-range rows, columns and k-chunks read as zero through the buffer
// descriptor's range check (an offset of 0x80000000 is never in range), so
// ragged M/N/K tails need no branches in the MAC loop (issue #1393 found the
// tile-change branches inside the K loop to be the main cost of its Triton
// Stream-K, so the segment walk lives outside the loop here).
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "schedule.h"

namespace gsk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int32_t s32x4 __attribute__((ext_vector_type(4)));
typedef int32_t s32x16 __attribute__((ext_vector_type(16)));

constexpr uint32_t kOutOfRange = 0x80000000u;
// Cache-policy operand of a buffer access that is coherent at agent scope
// (sc1): it neither hits a stale copy in this die's L2 nor leaves its write
// there.  Stream-K partials and flags cross dies through these, so the fixup
// needs no whole-L2 write-back or invalidate (an agent-scope fence costs every
// workgroup on the die its cached operand tiles).
constexpr int kAgentCoherent = 16;
// Buffer descriptor word 3 for gfx9-family raw (untyped, stride 0) buffers.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff,
                                             kRsrcWord3);
}

// Bits of a float, taken by value.  (A bit cast applied directly to one
// subscripted element of a vector lvalue was lowered to a read of element 0;
// every scalar reinterpretation in this file goes through here.)
__device__ __forceinline__ uint32_t bits_of(float x) { return __builtin_bit_cast(uint32_t, x); }

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, 0);
}

// Byte offset of 16-byte chunk `chunk` (0..7) of LDS row `row`.
__device__ __forceinline__ uint32_t lds_offset(int row, int chunk)
{
    return (uint32_t)(row * 128 + (((chunk ^ row ^ (row >> 3)) & 7) << 4));
}

template <int DT, int BM, int BN, int WM, int WN>
struct Tile {
    static constexpr int NTH = 64 * WM * WN;
    static constexpr int E = DT == 0 ? 4 : (DT == 3 ? 1 : 2); // bytes per element
    static constexpr int V = 16 / E;                  // elements per 16-byte chunk
    static constexpr int BK = 128 / E;                // k per MAC iteration (8 chunks)
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int MT = WTM / 32, NT = WTN / 32; // 32x32 blocks per wave
    static constexpr int A_LOADS = BM * 8 / NTH;      // 16-byte A chunks per thread
    static constexpr int B_LOADS = BK * BN / V / NTH; // 16-byte B chunks per thread
    static constexpr int R = B_LOADS < V ? B_LOADS : V; // k rows per transposed block
    static constexpr int NB = B_LOADS / R;            // transposed blocks per thread
    static constexpr int A_STAGE = BM * 128, B_STAGE = BN * 128;
    static constexpr int LDS = 2 * (A_STAGE + B_STAGE);
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(A_LOADS >= 1 && A_LOADS * NTH == BM * 8, "A slab must split evenly");
    static_assert(B_LOADS >= 2 && B_LOADS * NTH * V == BK * BN, "B slab must split evenly");
    static_assert(NB * R == B_LOADS && (R == 2 || R == 4 || R == 8), "B block shape");
    static_assert(R * E >= 4, "a transposed block must fill whole 32-bit words");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// One slab step (k = 2 chunks per lane pair) of a 32x32 block, operands swapped
// so the accumulator holds the transposed block.
template <int DT>
__device__ __forceinline__ void mfma_step(f32x16 &acc, const u32x4 &bt, const u32x4 &a)
{
    if constexpr (DT == 1) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, bt),
                                                     __builtin_bit_cast(f16x8, a), acc, 0, 0, 0);
    } else if constexpr (DT == 2) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bt),
                                                      __builtin_bit_cast(bf16x8, a), acc, 0, 0, 0);
    } else if constexpr (DT == 3) {
        // int8: 16 k per lane and operand, exact int32 sums kept in the
        // accumulator's 32-bit registers
        acc = __builtin_bit_cast(
            f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(s32x4, bt),
                                                          __builtin_bit_cast(s32x4, a),
                                                          __builtin_bit_cast(s32x16, acc), 0, 0,
                                                          0));
    } else {
        // fp32: a lane's chunk is 4 consecutive k; instruction e takes element e
        // from both operands, so the same k meets the same k.  (The whole vector
        // is reinterpreted first: a bit cast of one subscripted element of a
        // vector lvalue was lowered to a read of element 0.)
        const f32x4 btf = __builtin_bit_cast(f32x4, bt);
        const f32x4 af = __builtin_bit_cast(f32x4, a);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(btf[e], af[e], acc, 0, 0, 0);
    }
}

// Gather element v of each of the R rows in rows[] into one little-endian
// vector of R elements (the k-contiguous run for output column v).
template <int E, int R>
struct Transposed;

template <int R>
struct Transposed<2, R> {
    uint32_t w[R / 2];
    __device__ __forceinline__ void gather(const u32x4 *rows, int v)
    {
        const uint32_t sel = (v & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int j = 0; j < R / 2; ++j)
            w[j] = __builtin_amdgcn_perm(rows[2 * j + 1][v >> 1], rows[2 * j][v >> 1], sel);
    }
};

template <int R>
struct Transposed<1, R> {
    uint32_t w[R / 4];
    __device__ __forceinline__ void gather(const u32x4 *rows, int v)
    {
        // byte v&3 of word v>>2 of four rows -> one word, k ascending
        const uint32_t b = (uint32_t)(v & 3);
        const uint32_t sel = b | ((4u + b) << 8);
#pragma unroll
        for (int j = 0; j < R / 4; ++j) {
            const uint32_t lo = __builtin_amdgcn_perm(rows[4 * j + 1][v >> 2],
                                                      rows[4 * j][v >> 2], sel);
            const uint32_t hi = __builtin_amdgcn_perm(rows[4 * j + 3][v >> 2],
                                                      rows[4 * j + 2][v >> 2], sel);
            w[j] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        }
    }
};

template <int R>
struct Transposed<4, R> {
    uint32_t w[R];
    __device__ __forceinline__ void gather(const u32x4 *rows, int v)
    {
#pragma unroll
        for (int j = 0; j < R; ++j)
            w[j] = rows[j][v];
    }
};

template <int NWORDS>
__device__ __forceinline__ void lds_store_words(uint8_t *p, const uint32_t *w)
{
    if constexpr (NWORDS == 4) {
        *(u32x4 *)p = u32x4{w[0], w[1], w[2], w[3]};
    } else if constexpr (NWORDS == 2) {
        *(u32x2 *)p = u32x2{w[0], w[1]};
    } else {
        *(uint32_t *)p = w[0];
    }
}

// fp32 -> fp16 / bf16 bits, rounded to nearest even (by value: see bits_of).
__device__ __forceinline__ uint32_t f16_bits(float x)
{
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ uint32_t bf16_bits(float x)
{
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Store one 32x32 accumulator block (rows row0 + 32*mt.., columns col0 +
// 32*nt.. of the tile) to C through a buffer descriptor based at the tile's
// first row; an element outside C gets an out-of-range offset so its write is
// dropped: no branches around the stores.  C is fp32, or fp16 / bf16 rounded
// to nearest even from the fp32 sums (args.c_dtype, uniform per launch).
//
// A lane's four consecutive elements go out as one vector store when `vec`
// (uniform): the four are then either all inside C or all outside, which
// holds when N % 4 == 0 (args.c_vec) and in every tile that ends at or
// before column N.  The vector's address is only element-aligned when N % 4
// != 0; gfx950 runs with unaligned memory access enabled, as the repack's
// 16-byte loads from element-aligned rows also rely on.  Otherwise (the tile
// on the right edge of a C whose rows are not whole vectors) each element is
// stored on its own.
// (row: tile row; n: the first of the four columns of C)
__device__ __forceinline__ void store_quad_at(const f32x4 &v, const KernelArgs &args,
                                              __amdgpu_buffer_rsrc_t c_rsrc, int m0, int row, int n,
                                              bool vec)
{
    const bool row_ok = m0 + row < args.M;
    if (args.c_dtype != 0) {
        const uint32_t off = (uint32_t)((row * args.ldc + n) * 2);
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            h[e] = args.c_dtype == 1 ? f16_bits(v[e]) : bf16_bits(v[e]);
        if (vec) {
            const u32x2 u = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
            __builtin_amdgcn_raw_buffer_store_b64(
                u, c_rsrc, (int)(row_ok && n < args.N ? off : kOutOfRange), 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                __builtin_amdgcn_raw_buffer_store_b16(
                    (uint16_t)h[e], c_rsrc,
                    (int)(row_ok && n + e < args.N ? off + 2 * e : kOutOfRange), 0, 0);
        }
        return;
    }
    const uint32_t off = (uint32_t)((row * args.ldc + n) * 4);
    const u32x4 u = u32x4{bits_of(v[0]), bits_of(v[1]), bits_of(v[2]), bits_of(v[3])};
    if (vec) {
        // the vector is either wholly inside C or wholly outside
        __builtin_amdgcn_raw_buffer_store_b128(u, c_rsrc,
                                               (int)(row_ok && n < args.N ? off : kOutOfRange),
                                               0, 0);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(
                u[e], c_rsrc, (int)(row_ok && n + e < args.N ? off + 4 * e : kOutOfRange), 0, 0);
    }
}

// Quad g of the lane (row and half as in the accumulator layout).
__device__ __forceinline__ void store_quad(const f32x4 &v, const KernelArgs &args,
                                           __amdgpu_buffer_rsrc_t c_rsrc, int m0, int n0, int row,
                                           int col, int half, int g, bool vec)
{
    store_quad_at(v, args, c_rsrc, m0, row, n0 + col + 8 * g + 4 * half, vec);
}

// Descriptor for the C rows of a tile starting at row m0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t c_rows(const KernelArgs &args, int m0)
{
    return make_rsrc(args.C + (int64_t)m0 * args.ldc * (args.c_dtype != 0 ? 2 : 4));
}

// Quads 2j and 2j + 1 of one 32x32 block at tile rows brow.., columns col..
// (lane l holds row brow + l % 32 at columns 8g + 4(l / 32) .. + 3 in quad
// g).  As laid out, a store of one quad touches 32 rows with 32 bytes each.
// For vector stores the two quads are first exchanged with
// v_permlane16_swap, which swaps lanes 16-31 and 48-63 of quad 2j with lanes
// 0-15 and 32-47 of quad 2j + 1: afterwards quad 2j holds rows brow + (l % 16)
// and quad 2j + 1 rows brow + 16 + (l % 16), at columns 16j + 8((l / 16) % 2)
// + 4(l / 32) .. + 3, so each store covers 16 rows with 64 contiguous bytes
// (fp32 / int32 C; 32 bytes for 16-bit C): half the cache lines per store.
__device__ __forceinline__ void store_quad_pair(const f32x4 &q0, const f32x4 &q1,
                                                const KernelArgs &args,
                                                __amdgpu_buffer_rsrc_t c_rsrc, int m0, int n0,
                                                int brow, int col, int j, int lane, bool vec)
{
    if (vec) {
        f32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const auto r =
                __builtin_amdgcn_permlane16_swap(bits_of(q0[e]), bits_of(q1[e]), false, false);
            lo[e] = __builtin_bit_cast(float, (uint32_t)r[0]);
            hi[e] = __builtin_bit_cast(float, (uint32_t)r[1]);
        }
        const int r16 = lane & 15;
        const int n = n0 + col + 16 * j + 8 * ((lane >> 4) & 1) + 4 * (lane >> 5);
        store_quad_at(lo, args, c_rsrc, m0, brow + r16, n, true);
        store_quad_at(hi, args, c_rsrc, m0, brow + 16 + r16, n, true);
        return;
    }
    const int row = brow + (lane & 31), half = lane >> 5;
    store_quad(q0, args, c_rsrc, m0, n0, row, col, half, 2 * j, false);
    store_quad(q1, args, c_rsrc, m0, n0, row, col, half, 2 * j + 1, false);
}

__device__ __forceinline__ void store_block(const f32x16 &blk, const KernelArgs &args,
                                            __amdgpu_buffer_rsrc_t c_rsrc, int m0, int n0,
                                            int brow, int col, int lane, bool vec)
{
#pragma unroll
    for (int j = 0; j < 2; ++j)
        store_quad_pair(f32x4{blk[8 * j], blk[8 * j + 1], blk[8 * j + 2], blk[8 * j + 3]},
                        f32x4{blk[8 * j + 4], blk[8 * j + 5], blk[8 * j + 6], blk[8 * j + 7]},
                        args, c_rsrc, m0, n0, brow, col, j, lane, vec);
}

// Vector stores for a tile at columns n0 .. n0 + BN - 1 (see store_quad).
template <int BN>
__device__ __forceinline__ bool vector_stores(const KernelArgs &args, int n0)
{
    return args.c_vec || n0 + BN <= args.N;
}

// Wave 0 waits until the flags of workgroups q_first .. q_last are all set;
// slot_of(q) gives a workgroup's flag slot.  The lanes poll up to 64 flags at
// once, so many pieces cost one memory round trip, not one each.  With
// `clear`, each consumed flag is reset for the next run.  Bounded: after
// spin_limit rounds the status word is set and the wait gives up.
template <typename SlotOf>
__device__ __forceinline__ void wait_flags(const KernelArgs &args, int32_t q_first,
                                           int32_t q_last, SlotOf slot_of, bool clear)
{
    const int lane = threadIdx.x & 63;
    for (int32_t q0 = q_first; q0 <= q_last; q0 += 64) {
        const int32_t q = q0 + lane;
        const bool mine = q <= q_last;
        int32_t *flag = args.flags + (mine ? slot_of(q) : 0);
        int spins = 0;
        for (;;) {
            const bool ready =
                !mine || __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
            if (__builtin_amdgcn_ballot_w64(!ready) == 0)
                break;
            if (++spins > args.spin_limit) {
                if (lane == 0)
                    __hip_atomic_store(args.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (clear && mine)
            __hip_atomic_store(flag, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// a + b for two accumulator words: fp32 sums, or int32 sums carried in the
// same 32-bit registers (int8 inputs).  By value (see bits_of).
template <bool IACC>
__device__ __forceinline__ float acc_add(float a, float b)
{
    if constexpr (IACC)
        return __builtin_bit_cast(float, (int32_t)((uint32_t)__builtin_bit_cast(int32_t, a) +
                                                   (uint32_t)__builtin_bit_cast(int32_t, b)));
    else
        return a + b;
}

template <bool IACC>
__device__ __forceinline__ f32x4 acc_add4(const f32x4 &a, const f32x4 &b)
{
    if constexpr (IACC)
        return __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, a) + __builtin_bit_cast(u32x4, b));
    else
        return a + b;
}

// Finish one unit of work: a Stream-K tail is parked in the workgroup's
// partial slot and signalled; a split tile's head waits for its later
// workgroups and adds their partials; then the tile is stored to C.
//
// Accumulator layout (shared by both kernels): acc[mt][nt] is the 32x32 MFMA
// block at rows row0 + 32*mt, columns col0 + 32*nt of the tile, issued with
// swapped operands so that lane l holds C[row0 + 32*mt + l%32][col0 + 32*nt +
// 8*g + 4*(l/32) + e] in register 4*g + e.  A partial slot holds the blocks in
// this fragment order (lane-contiguous 16-byte vectors), so writes and reads of
// it are fully coalesced.  Partial slots are addressed through a buffer
// descriptor: lane offset in a VGPR and the fragment's offset as a scalar
// constant, so no per-fragment 64-bit addresses stay alive.
template <int BM, int BN, int MT, int NT, bool IACC = false>
__device__ __forceinline__ void finish_tile(f32x16 (&acc)[MT][NT], const KernelArgs &args,
                                            const WorkItem &w, int p, int m0, int n0, int wave,
                                            int lane, int row0, int col0)
{
    const int tid = threadIdx.x;
    const uint32_t lane_off = (uint32_t)lane * 16;
    if (w.role == ROLE_CONTRIB || (w.role == ROLE_OWNER && args.split_fixup)) {
        // A piece of a split tile: park it in this workgroup's slot, then
        // signal.  (With the split fixup the head piece is parked too, and the
        // tile's workgroups reduce it together after their MAC work.)
        const int32_t slot_id =
            args.split_fixup ? split_slot(p, w.role == ROLE_OWNER) : p;
        const __amdgpu_buffer_rsrc_t slot =
            make_rsrc(args.partials + (int64_t)slot_id * (BM * BN));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int f = ((wave * MT + mt) * NT + nt) * 4 + g;
                    const u32x4 u = u32x4{bits_of(acc[mt][nt][4 * g]),
                                          bits_of(acc[mt][nt][4 * g + 1]),
                                          bits_of(acc[mt][nt][4 * g + 2]),
                                          bits_of(acc[mt][nt][4 * g + 3])};
                    __builtin_amdgcn_raw_buffer_store_b128(u, slot, (int)lane_off, f * 1024,
                                                           kAgentCoherent);
                }
        // every lane's coherent stores have completed before the flag goes up
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0 && p != args.drop_signal_wg && args.split_fixup != 2)
            __hip_atomic_store(args.flags + slot_id, 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const __amdgpu_buffer_rsrc_t c_rsrc = c_rows(args, m0);
    const bool vec = vector_stores<BN>(args, n0);
    if (w.role == ROLE_OWNER) {
        // Head of a split tile: wait for every later workgroup on the tile,
        // then add their partials in ascending workgroup (= ascending k) order.
        // (consumed flags are cleared for the next run)
        if (wave == 0)
            wait_flags(args, p + 1, w.peer_last, [](int32_t q) { return q; }, true);
        // the partials are read below with agent-coherent loads issued after
        // the flags were seen
        __syncthreads();
        // Block by block: add the peers' partials in ascending order, store.
        const __amdgpu_buffer_rsrc_t slots = make_rsrc(args.partials);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x16 blk = acc[mt][nt];
                const uint32_t frag_off = (((wave * MT + mt) * NT + nt) * 4 * 64) * 16 + lane_off;
                for (int q = p + 1; q <= w.peer_last; ++q) {
                    // slot offsets stay below 2^31 bytes (g * bm * bn * 4 is checked at plan time)
                    const uint32_t off = (uint32_t)q * (uint32_t)(BM * BN * 4) + frag_off;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 v = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(slots, (int)off,
                                                                         g * 1024, kAgentCoherent));
                        blk[4 * g] = acc_add<IACC>(blk[4 * g], v[0]);
                        blk[4 * g + 1] = acc_add<IACC>(blk[4 * g + 1], v[1]);
                        blk[4 * g + 2] = acc_add<IACC>(blk[4 * g + 2], v[2]);
                        blk[4 * g + 3] = acc_add<IACC>(blk[4 * g + 3], v[3]);
                    }
                }
                store_block(blk, args, c_rsrc, m0, n0, row0 + mt * 32, col0 + nt * 32, lane,
                            vec);
            }
        return;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            store_block(acc[mt][nt], args, c_rsrc, m0, n0, row0 + mt * 32, col0 + nt * 32, lane,
                        vec);
}

// Reduce blocks [b0, b1) of split tile t (pieces of workgroups pf .. pl) and
// store them to C.  Every element adds the pieces in ascending k order (head
// piece first), the order the head's workgroup would use, so the result does
// not depend on who reduces.  Blocks are numbered in the writer's fragment
// order (wave, mt, nt); work units are half blocks (quads 2j and 2j + 1: 8
// values per lane, 2 KiB per piece) dealt to this workgroup's nwaves waves,
// and a unit's pieces are loaded QB at a time, all in flight together, then
// added in order.
template <int BM, int BN, int WM, int WN, bool IACC>
__device__ __forceinline__ void reduce_tile_blocks(const KernelArgs &args, int32_t t, int32_t pf,
                                                   int32_t pl, int32_t b0, int32_t b1, int wave,
                                                   int nwaves, int lane)
{
    constexpr int WTM = BM / WM, WTN = BN / WN, MT = WTM / 32, NT = WTN / 32;
    int tm, tn;
    tile_coords(args.P, t, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const __amdgpu_buffer_rsrc_t c_rsrc = c_rows(args, m0);
    const bool vec = vector_stores<BN>(args, n0);
    const __amdgpu_buffer_rsrc_t slots = make_rsrc(args.partials);
    const uint32_t slot_bytes = (uint32_t)(BM * BN * 4);
    constexpr int QB = 8;
    const int units = (b1 - b0) * 2;
    for (int u = wave; u < units; u += nwaves) {
        const int b = b0 + (u >> 1), j = u & 1;
        const int ww = b / (MT * NT), mt = (b / NT) % MT, nt = b % NT;
        const uint32_t frag_off = (uint32_t)(b * 4 * 64 + lane) * 16 + j * 2048;
        f32x4 s0 = f32x4{}, s1 = f32x4{};
        for (int32_t q0 = pf; q0 <= pl; q0 += QB) {
            f32x4 v[QB][2];
#pragma unroll
            for (int i = 0; i < QB; ++i)
                if (q0 + i <= pl) {
                    const int off =
                        (int)((uint32_t)split_slot(q0 + i, q0 + i == pf) * slot_bytes + frag_off);
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        v[i][h] = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(slots, off, h * 1024,
                                                                         kAgentCoherent));
                }
#pragma unroll
            for (int i = 0; i < QB; ++i)
                if (q0 + i <= pl) {
                    s0 = q0 + i == pf ? v[i][0] : acc_add4<IACC>(s0, v[i][0]);
                    s1 = q0 + i == pf ? v[i][1] : acc_add4<IACC>(s1, v[i][1]);
                }
        }
        store_quad_pair(s0, s1, args, c_rsrc, m0, n0, (ww / WN) * WTM + mt * 32,
                        (ww % WN) * WTN + nt * 32, j, lane, vec);
    }
}

// Split fixup, after the workgroup's MAC work: for each split tile it took
// part in, wait for all of the tile's pieces and reduce its share of the
// tile's 32x32 blocks.  The last workgroup to finish with a tile clears its
// flags and counter.
template <int BM, int BN, int WM, int WN, bool IACC = false>
__device__ __forceinline__ void reduce_split_tiles(const KernelArgs &args, int p, int wave,
                                                   int lane)
{
    constexpr int WTM = BM / WM, WTN = BN / WN, MT = WTM / 32, NT = WTN / 32;
    constexpr int NW = WM * WN, NBLK = NW * MT * NT;
    const Partition &P = args.P;
    const int tid = threadIdx.x;
    int32_t tiles[2];
    const int ntiles = split_tiles_of(P, p, tiles);
    for (int it = 0; it < ntiles; ++it) {
        const int32_t t = tiles[it];
        int32_t pf, pl;
        tile_workers(P, t, &pf, &pl);
        const int32_t parts = pl - pf + 1;
        int32_t b0, b1;
        split_share(p - pf, parts, NBLK, &b0, &b1);
        if (wave == 0)
            wait_flags(args, pf, pl, [pf](int32_t q) { return split_slot(q, q == pf); }, false);
        __syncthreads();
        reduce_tile_blocks<BM, BN, WM, WN, IACC>(args, t, pf, pl, b0, b1, wave, NW, lane);
        // this workgroup's reads of the tile's slots are complete (their values
        // are already summed) before it counts itself done
        __syncthreads();
        if (tid == 0) {
            const int32_t done = __hip_atomic_fetch_add(args.counters + t, 1, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            if (done == parts - 1) {
                // every reader of this tile is finished: leave it clean for the next run
                for (int32_t q = pf; q <= pl; ++q)
                    __hip_atomic_store(args.flags + split_slot(q, q == pf), 0, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(args.counters + t, 0, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// Two-kernel fixup (no waits, so no co-residency needed): launched after the
// GEMM kernel, one workgroup per Stream-K tile reduces all of a split tile's
// parked pieces in ascending k order and stores it.
template <int BM, int BN, int WM, int WN, bool IACC>
__global__ __launch_bounds__(64 * WM * WN, 1) void fixup_kernel(KernelArgs args)
{
    constexpr int WTM = BM / WM, WTN = BN / WN, MT = WTM / 32, NT = WTN / 32;
    constexpr int NW = WM * WN, NBLK = NW * MT * NT;
    const int32_t t = (int32_t)blockIdx.x;
    int32_t pf, pl;
    tile_workers(args.P, t, &pf, &pl);
    if (pf == pl)
        return;  // a whole tile: its workgroup stored it
    reduce_tile_blocks<BM, BN, WM, WN, IACC>(args, t, pf, pl, 0, NBLK, threadIdx.x >> 6, NW,
                                             threadIdx.x & 63);
}

template <int BM, int BN, int WM, int WN, bool IACC>
static int launch_fixup(const KernelArgs &args, int grid, hipStream_t stream)
{
    if (grid <= 0)
        return 0;
    hipLaunchKernelGGL((fixup_kernel<BM, BN, WM, WN, IACC>), dim3(grid), dim3(64 * WM * WN), 0,
                       stream, args);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// ---------------------------------------------------------------------------
// Register-staged kernel (fp32, int8, and fp16/bf16 at 64x64 tiles).
//
// One MAC iteration consumes a BK-deep slab of A (BM x BK) and B (BK x BN),
// BK being 128 bytes of input per row (32 fp32 or 64 fp16/bf16 values).  Slabs
// go global -> registers -> LDS with two LDS buffers, so the loads of slab
// k + 1 are in flight while slab k is multiplied, with one barrier per
// iteration ("double-buffering" in the persistent matmul post on the Hugging
// Face activity feed page).  Both operands sit in LDS as 128-byte rows with k
// contiguous (B is transposed in registers on its way in), chunk-swizzled with
// (row ^ row >> 3) & 7, so every MFMA operand is one 16-byte LDS read.
template <int DT, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_kernel(KernelArgs args)
{
    using Cfg = Tile<DT, BM, BN, WM, WN>;
    constexpr int NTH = Cfg::NTH, E = Cfg::E, V = Cfg::V, BK = Cfg::BK;
    constexpr int MT = Cfg::MT, NT = Cfg::NT, R = Cfg::R, NB = Cfg::NB;
    constexpr int A_LOADS = Cfg::A_LOADS;

    __shared__ __attribute__((aligned(16))) uint8_t lds[Cfg::LDS];

    const Partition &P = args.P;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wy = wave / WN, wx = wave - (wave / WN) * WN;
    const int half = lane >> 5, l32 = lane & 31;
    const int p = logical_wg((int32_t)blockIdx.x, P.grid, P.xcds);

    // Per-thread slab load coordinates (constant for the whole kernel).
    int a_row[A_LOADS], a_chunk[A_LOADS];
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
        int L = i * NTH + tid;
        a_row[i] = L >> 3;
        a_chunk[i] = L & 7;
    }
    constexpr int NCH = BN / V;  // 16-byte chunks across one B row of the tile
    int b_kg[NB], b_nc[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        int b = i * NTH + tid;
        b_nc[i] = b % NCH;
        b_kg[i] = b / NCH;
    }

    u32x4 ra[A_LOADS];
    u32x4 rb[NB][R];
    f32x16 acc[MT][NT];

    WorkCursor cur = work_begin(P, p);
    WorkItem w;
    while (work_next(P, p, cur, w)) {
        int tm, tn;
        tile_coords(P, w.tile, &tm, &tn);
        const int m0 = tm * BM, n0 = tn * BN;

        bool a_row_ok[A_LOADS];
        uint32_t a_off[A_LOADS];
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            a_row_ok[i] = m0 + a_row[i] < args.M;
            a_off[i] = (uint32_t)(a_row[i] * args.lda * E + a_chunk[i] * 16);
        }
        bool b_col_ok[NB];
        uint32_t b_off[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            b_col_ok[i] = n0 + b_nc[i] * V < args.N;
            b_off[i] = (uint32_t)(b_kg[i] * R * args.ldb * E + b_nc[i] * 16);
        }

        // Global -> registers for MAC iteration kk of this tile.
        auto load_slab = [&](int kk) {
            const int k0 = kk * BK;
            const __amdgpu_buffer_rsrc_t ra_rsrc =
                make_rsrc(args.A + ((int64_t)m0 * args.lda + k0) * E);
            const __amdgpu_buffer_rsrc_t rb_rsrc =
                make_rsrc(args.B + ((int64_t)k0 * args.ldb + n0) * E);
            const int k_left = args.K - k0;
#pragma unroll
            for (int i = 0; i < A_LOADS; ++i) {
                bool ok = a_row_ok[i] && a_chunk[i] * V < k_left;
                ra[i] = load16(ra_rsrc, ok ? a_off[i] : kOutOfRange);
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) {
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    bool ok = b_col_ok[i] && b_kg[i] * R + j < k_left;
                    rb[i][j] = load16(rb_rsrc, ok ? b_off[i] + (uint32_t)(j * args.ldb * E)
                                                  : kOutOfRange);
                }
            }
        };

        // Registers -> LDS stage s (B transposed to k-contiguous rows).
        auto store_slab = [&](int s) {
            uint8_t *As = lds + s * Cfg::A_STAGE;
            uint8_t *Bs = lds + 2 * Cfg::A_STAGE + s * Cfg::B_STAGE;
#pragma unroll
            for (int i = 0; i < A_LOADS; ++i)
                *(u32x4 *)(As + lds_offset(a_row[i], a_chunk[i])) = ra[i];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int kfirst = b_kg[i] * R;           // first k of the block
                const int chunk = kfirst / V, within = (kfirst % V) * E;
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    Transposed<E, R> t;
                    t.gather(rb[i], v);
                    const int row = b_nc[i] * V + v;
                    lds_store_words<R * E / 4>(Bs + lds_offset(row, chunk) + within, t.w);
                }
            }
        };

        // MFMAs over LDS stage s.
        auto compute_slab = [&](int s) {
            const uint8_t *As = lds + s * Cfg::A_STAGE;
            const uint8_t *Bs = lds + 2 * Cfg::A_STAGE + s * Cfg::B_STAGE;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                u32x4 af[MT], bf[NT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    af[mt] = *(const u32x4 *)(As + lds_offset(wy * Cfg::WTM + mt * 32 + l32,
                                                              2 * st + half));
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    bf[nt] = *(const u32x4 *)(Bs + lds_offset(wx * Cfg::WTN + nt * 32 + l32,
                                                              2 * st + half));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        mfma_step<DT>(acc[mt][nt], bf[nt], af[mt]);
            }
        };

#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[mt][nt] = f32x16{};

        load_slab(w.kb);
        __syncthreads();  // the previous item's last LDS reads are done
        store_slab(0);
        __syncthreads();
        int s = 0;
        for (int kk = w.kb; kk + 1 < w.ke; ++kk) {
            load_slab(kk + 1);
            // Keep the next slab's global loads at the top of the iteration so
            // their latency overlaps this slab's MFMAs (the scheduler would
            // otherwise sink them next to the LDS writes that consume them).
            __builtin_amdgcn_sched_barrier(0);
            compute_slab(s);
            store_slab(s ^ 1);
            __syncthreads();
            s ^= 1;
        }
        compute_slab(s);

        finish_tile<BM, BN, MT, NT, DT == 3>(acc, args, w, p, m0, n0, wave, lane,
                                             wy * Cfg::WTM, wx * Cfg::WTN);
    }
    if (args.split_fixup == 1)
        reduce_split_tiles<BM, BN, WM, WN, DT == 3>(args, p, wave, lane);
}

// ---------------------------------------------------------------------------
// Helpers of the direct-to-LDS kernel below.
//
// B sits in LDS row-major as in memory (k-rows of BN values) and is read
// with the transposing LDS read: each 16-lane group turns a 4 x 16 block of
// row-major values into per-lane runs of 4 k.  The 16-byte chunks of k-row r
// are XOR-swizzled with kB[r & 3], kB = {0, 6, 10, 12}, so the four k-rows a
// transposing read touches (32 bytes each per 16-lane group) hit distinct
// banks.
__device__ __forceinline__ uint32_t swz_b(int krow)
{
    return (0xCA60u >> ((krow & 3) * 4)) & 0xF;  // {0, 6, 10, 12}[krow & 3]
}

// int8 B (256-byte k-rows, read with ds_read_b64_tr_b8): chunk c of k-row r
// sits at c ^ 2*(r & 7).  A 32-lane half of a read touches 8 k-rows at two
// adjacent chunks (even c, c + 1), in both 8-byte halves: the 8 distinct
// even offsets 2*(r & 7) put the 32 reads on 32 distinct 8-byte bank pairs.
__device__ __forceinline__ uint32_t swz_b8(int krow) { return (uint32_t)(krow & 7) << 1; }

__device__ __forceinline__ void barrier_only()
{
    // A workgroup barrier with no memory fence: the copies it orders are
    // already complete (s_waitcnt above); the asm keeps the compiler from
    // moving LDS accesses across it.
    asm volatile("s_barrier" ::: "memory");
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int s32x2 __attribute__((ext_vector_type(2)));
#define GSK_LDS(T, p) ((__attribute__((address_space(3))) T *)(p))

// Raw buffer descriptor (base, no stride, 2^31 - 1 bytes, untyped) as four
// scalar words, for the copy issued from inline assembly below.
__device__ __forceinline__ i32x4 rsrc_words(const void *base)
{
    const uint64_t b = (uint64_t)base;
    return i32x4{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xffff), 0x7fffffff, kRsrcWord3};
}

// Copy 16 bytes per lane from buffer offset voff (0x80000000: out of range,
// zeros) into LDS at lds_addr + 16 * lane (lds_addr wave-uniform).  Issued as
// inline assembly so that the compiler does not treat it as an outstanding LDS
// write: it would otherwise wait for every copy in flight before each
// transposing LDS read, which defeats the ring.  The ring's own s_waitcnt
// vmcnt() waits and barriers order these copies against the reads.
// STREAM adds the non-temporal hint: the lines are not kept for reuse in the
// caches, which pays where each operand line is read by few workgroups at once
// (few tiles, long K) and costs where tiles share panels in L2.
template <bool STREAM = false>
__device__ __forceinline__ void copy16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %0\n\t"
                     "s_nop 0\n\t"
                     "buffer_load_dwordx4 %1, %2, 0 offen nt lds"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc)
                     : "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\t"
                     "s_nop 0\n\t"
                     "buffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc)
                     : "m0");
}

__device__ __forceinline__ uint32_t lds_address(const uint8_t *p)
{
    return (uint32_t)(uintptr_t)GSK_LDS(const uint8_t, p);
}

template <int V>
struct IC {
    static constexpr int value = V;
};

// f(IC<B>{}), f(IC<B+1>{}), ..., f(IC<E-1>{}): a loop whose index is a
// compile-time constant in the body.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(IC<B>{});
        static_for<B + 1, E>(f);
    }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------
// fp16/bf16 kernel with direct global -> LDS loads, A copied in whole rows.
//
// A MAC iteration is 64 deep (BK = 64): its A slab is BM rows of 128 bytes,
// whole cache lines, and it is multiplied as two 32-deep halves.  (Copying A
// in 64-byte row halves, an iteration apart, fetched every A line twice
// through the vector L1; on a 4096^3 product that made the pure load phase
// ~20% slower.)  A fragments are 16-byte LDS reads of k-contiguous rows; B
// fragments come from the transposing LDS read, so neither operand passes
// through registers on its way into LDS.
//
// LDS: four B stages (one per half-iteration: 32 k-rows x BN values,
// swizzled with swz_b) followed by three A slots (one per iteration: BM rows
// x 128 bytes, 16-byte chunk c of row r at position c ^ ((r ^ r >> 3) & 7)).
//
// Copy schedule in half-iterations t of the segment: half-iteration t issues
// the B slab of t + 3 and half (t & 1) of the A slab of iteration (t >> 1) + 2
// (half 0 = rows [0, BM/2), half 1 = rows [BM/2, BM)), so every copy lands at
// least three half-iterations before its first use.  The A slab goes into
// the slot of iteration (t >> 1) - 1, whose last half is t - 1, and B slab
// t + 3 into the stage of t - 1: both are free once every wave has passed the
// barrier in the middle of half-iteration t.  The segment starts with the
// copies that half-iterations -4 .. -1 would have issued.  Copies past the
// end of the segment read nothing (out-of-range offsets) and fill a free slot
// or stage with zeros, so every half-iteration issues the same number of
// copies and every wait count is a constant.
template <int DT, int BM, int BN, int WM, int WN>
struct PairTile {
    static constexpr int NW = WM * WN, NTH = 64 * NW;
    static constexpr int E = DT == 3 ? 1 : 2;              // bytes per element
    static constexpr int V = 16 / E;                       // elements per 16-byte chunk
    // iteration and half depth: one 128-byte A row segment per iteration
    static constexpr int BK = 128 / E, HK = 64 / E;
    static constexpr int SA = 3, SB = 4;                   // A slots, B stages
    static constexpr int B_ROW = BN * E;                   // bytes per B k-row
    static constexpr int A_SLOT = BM * 128, B_STAGE = HK * BN * E;
    static constexpr int A_BASE = SB * B_STAGE;
    static constexpr int LDS = SB * B_STAGE + SA * A_SLOT;
    static constexpr int A_INSTR = A_SLOT / 2 / 1024 / NW; // 1 KiB copies per wave and half slab
    static constexpr int B_INSTR = B_STAGE / 1024 / NW;
    static constexpr int LPI = A_INSTR + B_INSTR;          // copies per wave and half-iteration
    static constexpr int WTM = BM / WM, WTN = BN / WN, MT = WTM / 32, NT = WTN / 32;
    static_assert(DT == 1 || DT == 2 || DT == 3, "fp16 / bf16 / int8 only");
    static_assert(A_INSTR >= 1 && A_INSTR * 2 * 1024 * NW == A_SLOT &&
                      B_INSTR >= 1 && B_INSTR * 1024 * NW == B_STAGE,
                  "copies must split evenly over the waves");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0 && BN >= 128, "tile shape");
    static_assert(2 * LPI <= 63, "wait counts");
    static_assert(MT * NT >= LPI, "one copy per MFMA of a slab");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ uint32_t swz_row128(int row) { return (uint32_t)(row ^ (row >> 3)) & 7; }

template <int DT, int BM, int BN, int WM, int WN, bool STREAM = false>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_kernel_pair(KernelArgs args)
{
    using Cfg = PairTile<DT, BM, BN, WM, WN>;
    constexpr int NW = Cfg::NW, MT = Cfg::MT, NT = Cfg::NT, HK = Cfg::HK;
    constexpr int A_INSTR = Cfg::A_INSTR, B_INSTR = Cfg::B_INSTR, LPI = Cfg::LPI;
    constexpr int A_SLOT = Cfg::A_SLOT, B_STAGE = Cfg::B_STAGE, A_BASE = Cfg::A_BASE;
    constexpr int B_ROW = Cfg::B_ROW, SA = Cfg::SA, SB = Cfg::SB;
    constexpr int NMFMA = MT * NT;  // MFMAs per slab
    constexpr int NREAD = MT + NT;  // fragment reads per slab
    static_assert(2 * NMFMA >= NREAD, "two fragment reads per MFMA");
    static_assert(DT == 1 || DT == 2, "the ring kernel's B layout is for 16-bit elements");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[Cfg::LDS];

    const Partition &P = args.P;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wy = wave / WN, wx = wave - (wave / WN) * WN;
    const int half = lane >> 5, l32 = lane & 31;
    const int p = logical_wg((int32_t)blockIdx.x, P.grid, P.xcds);
    const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds_address(lds) + wave * 1024);

    // A copy jj (0 .. 2*A_INSTR-1; half h issues jj in [h*A_INSTR, (h+1)*A_INSTR))
    // fills 1 KiB block jj*NW + wave of a slot: 8 rows of 128 bytes, the lane
    // writing position lane & 7 of row 8*block + lane/8.
    auto a_copy_row = [&](int jj) { return (jj * NW + wave) * 8 + (lane >> 3); };
    int b_krow[B_INSTR], b_chunk[B_INSTR];
#pragma unroll
    for (int j = 0; j < B_INSTR; ++j) {
        const int o = (j * NW + wave) * 1024 + lane * 16;
        b_krow[j] = o / B_ROW;
        b_chunk[j] = ((o % B_ROW) >> 4) ^ swz_b(o / B_ROW);
    }

    // Fragment read addresses.  A: the lane's row r0 = wy*WTM + l32 at chunk
    // `half` (slab 0 of the first half-iteration).  Slab 1 is chunk + 2, the
    // second half-iteration chunk + 4, and block mt + 1 is 32 rows on, which
    // flips bit 2 of the row's swizzle: bits 5 and 6 of the byte offset (XOR)
    // and 4 KiB steps (add).  B: the lane's transposing-read address for
    // k-rows 8*(g/2) + si/4 of block nt; the other three reads of the block
    // (4 and 16 k-rows on) keep the swizzle, which depends on the k-row mod 4
    // only.  Stage s adds s times the stage size, so every read is a base
    // register plus a constant.
    const int r0 = wy * Cfg::WTM + l32;
    const uint32_t a_lane = A_BASE + (uint32_t)(r0 * 128) + ((half ^ swz_row128(r0)) << 4);
    uint32_t b_rd[NT];
    {
        const int g = lane >> 4, si = lane & 15;
        const int krow = 8 * (g >> 1) + (si >> 2);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n = wx * Cfg::WTN + nt * 32 + 16 * (g & 1) + 4 * (si & 3);
            b_rd[nt] = krow * B_ROW + (((n >> 3) ^ swz_b(krow)) << 4) + (n & 7) * 2;
        }
    }
    // slot_off: A slot byte offset (runtime); odd, st, s: compile-time
    auto read_a = [&](uint32_t slot_off, int odd, int st, int mt) {
        const uint32_t x = (uint32_t)((st << 5) | ((odd ^ (mt & 1)) << 6));
        return *(const u32x4 *)(lds + slot_off + mt * 4096 + (a_lane ^ x));
    };
    auto read_b = [&](int s, int st, int nt) {
        const uint8_t *base = lds + b_rd[nt] + s * B_STAGE + st * 16 * B_ROW;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(GSK_LDS(i16x4, base));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(GSK_LDS(i16x4, base + 4 * B_ROW));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };
    // Fragment read r of a slab in the order its MFMAs first need them.
    auto read_frag = [&](uint32_t slot_off, int odd, int s, int st, int r, u32x4 (&fa)[MT],
                         u32x4 (&fb)[NT]) {
        if (r == 0)
            fa[0] = read_a(slot_off, odd, st, 0);
        else if (r <= NT)
            fb[r - 1] = read_b(s, st, r - 1);
        else
            fa[r - NT] = read_a(slot_off, odd, st, r - NT);
    };

    f32x16 acc[MT][NT];
    u32x4 fa0[MT], fb0[NT], fa1[MT], fb1[NT];

    WorkCursor cur = work_begin(P, p);
    WorkItem w;
    while (work_next(P, p, cur, w)) {
        int tm, tn;
        tile_coords(P, w.tile, &tm, &tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const int k_lo = w.kb * Cfg::BK;
        const int k_hi = w.ke * Cfg::BK < args.K ? w.ke * Cfg::BK : args.K;
        const int n = (k_hi - k_lo + HK - 1) / HK;  // half-iterations of this item (>= 1)

        uint32_t a_off[2 * A_INSTR];
#pragma unroll
        for (int jj = 0; jj < 2 * A_INSTR; ++jj) {
            const int row = a_copy_row(jj);
            a_off[jj] = m0 + row < args.M
                            ? (uint32_t)(row * args.lda * 2 +
                                         (((lane & 7) ^ (int)swz_row128(row)) << 4))
                            : kOutOfRange;
        }
        uint32_t b_off[B_INSTR];
#pragma unroll
        for (int j = 0; j < B_INSTR; ++j)
            b_off[j] = n0 + b_chunk[j] * 8 < args.N
                           ? (uint32_t)(b_krow[j] * args.ldb * 2 + b_chunk[j] * 16)
                           : kOutOfRange;

        // Next A slab to copy (its k and source; the pointer stops at the
        // item's last slab) and next B half-slab (likewise).
        int ka = k_lo;
        const uint8_t *a_cp = args.A + ((int64_t)m0 * args.lda + k_lo) * 2;
        int kbh = k_lo;
        const uint8_t *b_cp = args.B + ((int64_t)k_lo * args.ldb + n0) * 2;
        const int64_t b_step = (int64_t)HK * args.ldb * 2;

        // Copies of one half-iteration: half h of the next A slab into slot
        // `a_slot`, then the next B half-slab into stage s_fill.
        auto copy_a = [&](int h, uint32_t a_slot_off, int j) {
            const int jj = h * A_INSTR + j;
            const bool whole = ka + Cfg::BK <= k_hi;
            const int chunk = (lane & 7) ^ (int)swz_row128(a_copy_row(jj));
            const uint32_t off = whole || chunk * 8 < k_hi - ka ? a_off[jj] : kOutOfRange;
            copy16<STREAM>(rsrc_words(a_cp), off, lds_wave + A_BASE + a_slot_off + jj * NW * 1024);
        };
        auto next_a = [&]() {
            if (ka + Cfg::BK < k_hi)
                a_cp += Cfg::BK * 2;
            ka += Cfg::BK;
        };
        auto copy_b = [&](int s_fill, int j) {
            const bool whole = kbh + HK <= k_hi;
            const uint32_t off = whole || b_krow[j] < k_hi - kbh ? b_off[j] : kOutOfRange;
            copy16<STREAM>(rsrc_words(b_cp), off, lds_wave + s_fill * B_STAGE + j * NW * 1024);
        };
        auto next_b = [&]() {
            if (kbh + HK < k_hi)
                b_cp += b_step;
            kbh += HK;
        };

#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[mt][nt] = f32x16{};

        // All waves are done with the previous item's slots before refilling.
        barrier_only();
        // half-iterations -4 .. -1: A slabs 0 and 1 into slots 0 and 1, B
        // half-slabs -1 (nothing to read) .. 2 into stages 3, 0, 1, 2
        static_for<0, 4>([&](auto u) {
            constexpr int h = u.value & 1;
#pragma unroll
            for (int j = 0; j < A_INSTR; ++j)
                copy_a(h, (u.value >> 1) * A_SLOT, j);
            if (h)
                next_a();
            if constexpr (u.value == 0) {
                // half-slab -1: nothing to read, a zero fill keeps the count
#pragma unroll
                for (int j = 0; j < B_INSTR; ++j)
                    copy16<STREAM>(rsrc_words(b_cp), kOutOfRange,
                           lds_wave + (SB - 1) * B_STAGE + j * NW * 1024);
            } else {
#pragma unroll
                for (int j = 0; j < B_INSTR; ++j)
                    copy_b(u.value - 1, j);
                next_b();
            }
        });
        wait_vmcnt<2 * LPI>();  // half-iteration 0's copies have landed
        barrier_only();

        uint32_t sa_off = 0;             // slot of the current A slab
        uint32_t fill_off = 2 * A_SLOT;  // slot of the slab two ahead
#pragma unroll
        for (int r = 0; r < NREAD; ++r)
            read_frag(sa_off, 0, 0, 0, r, fa0, fb0);

        // Half-iteration t (B stage t mod 4 and parity t mod 2 are
        // compile-time constants here); `surely_more` says at compile time
        // that another half-iteration follows.
        auto step = [&](int t, auto u_c, auto surely_more) {
            constexpr int u = decltype(u_c)::value;
            constexpr int odd = u & 1, s = u & (SB - 1);
            constexpr int s_next = (s + 1) & (SB - 1), s_fill = (s + SB - 1) & (SB - 1);
            const uint32_t sa_next = odd ? (sa_off + A_SLOT == SA * A_SLOT ? 0 : sa_off + A_SLOT)
                                         : sa_off;
            // (a) first slab's MFMAs, the second slab's reads between
#pragma unroll
            for (int j = 0; j < NMFMA; ++j) {
                mfma_step<DT>(acc[j / NT][j % NT], fb0[j % NT], fa0[j / NT]);
#pragma unroll
                for (int r = 2 * j; r < 2 * j + 2 && r < NREAD; ++r)
                    read_frag(sa_off, odd, s, 1, r, fa1, fb1);
                __builtin_amdgcn_sched_barrier(0);
            }
            const bool more = decltype(surely_more)::value || t + 1 < n;
            if (more) {
                // (b) half-iteration t + 1's copies are complete in every wave
                //     (only those of t - 1 may be in flight), and every wave
                //     is past t - 1's slot and stage
                wait_vmcnt<LPI>();
                barrier_only();
            }
            // (c) second slab's MFMAs, with the next half-iteration's
            //     first-slab reads and this half-iteration's copies (none on
            //     the last one: without the barrier others may still read)
#pragma unroll
            for (int j = 0; j < NMFMA; ++j) {
                mfma_step<DT>(acc[j / NT][j % NT], fb1[j % NT], fa1[j / NT]);
#pragma unroll
                for (int r = 2 * j; r < 2 * j + 2 && r < NREAD; ++r)
                    read_frag(sa_next, odd ^ 1, s_next, 0, r, fa0, fb0);
                if (more && j >= NMFMA - LPI) {
                    const int c = j - (NMFMA - LPI);
                    if (c < A_INSTR)
                        copy_a(odd, fill_off, c);
                    else
                        copy_b(s_fill, c - A_INSTR);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (more) {
                if (odd) {
                    next_a();
                    fill_off = fill_off + A_SLOT == SA * A_SLOT ? 0 : fill_off + A_SLOT;
                }
                next_b();
            }
            sa_off = sa_next;
        };
        int t = 0;
        for (; t + SB <= n; t += SB)
            static_for<0, SB>([&](auto u) { step(t + u.value, u, IC<(u.value < SB - 1)>{}); });
        static_for<0, SB - 1>([&](auto u) {
            if (t + u.value < n)
                step(t + u.value, u, IC<0>{});
        });

        finish_tile<BM, BN, MT, NT>(acc, args, w, p, m0, n0, wave, lane, wy * Cfg::WTM,
                                    wx * Cfg::WTN);
    }
    if (args.split_fixup == 1)
        reduce_split_tiles<BM, BN, WM, WN>(args, p, wave, lane);
}

// ---------------------------------------------------------------------------
// fp16/bf16 wave-specialised "ping-pong" kernel (256x256 tiles, 8 waves).
//
// The waves form two groups of four, one wave of each group on every SIMD
// (wave w runs on SIMD w mod 4): group 0 (waves 0-3) computes tile rows
// 0-127, group 1 (waves 4-7) rows 128-255, each wave a 128 x 64 block.  Time
// is cut into phases separated by workgroup barriers, and the groups take
// turns: while one group runs a burst of 16 MFMAs on fragments it already
// holds in registers, the other does its memory work for its next burst (its
// share of the global -> LDS copies, the LDS fragment reads, and the waits),
// so each SIMD's matrix unit is fed by one wave while the other waits on
// memory.  With half-iterations h (32 k each):
//   phase 2h:     group 0 multiplies h;       group 1 reads h
//   phase 2h + 1: group 0 reads h + 1;        group 1 multiplies h
// (group 0 reads h = 0 in a phase of its own before phase 0).
//
// Copies: in its memory phase for h, group 1 copies the B stage of h + 3 and
// group 0 the A rows of h + 3 (rows 0-127 of iteration (h + 3) >> 1 when h + 3
// is even, rows 128-255 when it is odd); each is 16 KiB, four 1 KiB copies
// per wave.  The item starts with the copies of h = 0, 1, 2.  Every wave waits
// at the end of every phase until at most two of its copy batches are in
// flight, so each copy has two phases' worth of time to land.  The LDS layout
// is gemm_kernel_pair's (four B stages of 32 k-rows, three A slots of 64 k),
// and a CPU model of this schedule (every read sees landed data; no copy
// overwrites a buffer still being read, copies past the end included) was
// checked for every segment length up to 199 half-iterations.  As in
// gemm_kernel_pair, copies past the end of a segment read nothing and zero a
// free buffer, so the wait counts are constants.
//
// Accumulators, the epilogue and the Stream-K fixups are gemm_kernel_pair's
// with the 2 x 4 wave layout (group = wave row, wave mod 4 = wave column).
// The body run by one group (GRP 0 or 1).  Each group has its own copy of
// the whole work loop, so no register value is merged between the groups'
// paths; both copies cross the same barriers in the same order.
template <int DT, int GRP>
__device__ __forceinline__ void gemm_pp_group(const KernelArgs &args, uint8_t *lds, int q,
                                              int lane, int p)
{
    using Cfg = PairTile<DT, 256, 256, 2, 4>;
    constexpr int MT = Cfg::MT, NT = Cfg::NT, HK = Cfg::HK, BK = Cfg::BK;
    constexpr int A_SLOT = Cfg::A_SLOT, B_STAGE = Cfg::B_STAGE, A_BASE = Cfg::A_BASE;
    constexpr int B_ROW = Cfg::B_ROW, SB = Cfg::SB, SA = Cfg::SA;
    constexpr int E = Cfg::E, V = Cfg::V;  // bytes per element, elements per 16-byte chunk
    static_assert(MT == 4 && NT == 2 && SB == 4 && SA == 3, "256x256, 2x4 waves");
    const Partition &P = args.P;
    const int wave = GRP * 4 + q;
    const int half = lane >> 5, l32 = lane & 31;
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_address(lds));

    // Copy geometry.  Copy j (0..3) of this wave fills 1 KiB block 4j + q of a
    // 16 KiB piece.  Group 0: rows 8*(4j + q) + lane/8 of the A row half,
    // position lane & 7 holding 16-byte chunk (lane & 7) ^ swizzle(row) (the
    // swizzle is the same for both row halves: they differ by 128 rows).
    // Group 1: k-rows 2*(4j + q) + lane/32 of the B stage (512-byte rows of
    // 16-bit elements), or 4*(4j + q) + lane/16 (256-byte rows of int8), each
    // position holding the swizzled 16-byte chunk of its row (swz_b, swz_b8).
    int cp_row[4], cp_chunk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (GRP == 0) {
            cp_row[j] = 8 * (4 * j + q) + (lane >> 3);
            cp_chunk[j] = (lane & 7) ^ (int)swz_row128(cp_row[j]);
        } else if constexpr (E == 2) {
            cp_row[j] = 2 * (4 * j + q) + (lane >> 5);
            cp_chunk[j] = (lane & 31) ^ (int)swz_b(cp_row[j]);
        } else {
            cp_row[j] = 4 * (4 * j + q) + (lane >> 4);
            cp_chunk[j] = (lane & 15) ^ (int)swz_b8(cp_row[j]);
        }
    }
    const uint32_t cp_lds = lds_base + (uint32_t)q * 1024;

    // Fragment read addresses (gemm_kernel_pair's, with wave row GRP and
    // wave column q).
    const int r0 = GRP * Cfg::WTM + l32;
    const uint32_t a_lane = A_BASE + (uint32_t)(r0 * 128) + ((half ^ swz_row128(r0)) << 4);
    uint32_t b_rd[NT];
    if constexpr (E == 2) {
        const int g = lane >> 4, si = lane & 15;
        const int krow = 8 * (g >> 1) + (si >> 2);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n = q * Cfg::WTN + nt * 32 + 16 * (g & 1) + 4 * (si & 3);
            b_rd[nt] = krow * B_ROW + (((n >> 3) ^ swz_b(krow)) << 4) + (n & 7) * 2;
        }
    } else {
        // int8 (ds_read_b64_tr_b8): within each 16-lane group, lane i receives
        // byte i % 8 of the 8-byte chunks that source lanes 2j + i / 8 (j = 0..7)
        // address.  Source lane s of group g points at k-row 16*(g/2) + s/2 and
        // columns 16*(g%2) + 8*(s%2) .. + 7 of the wave's 32-column block, so
        // lane i of the group gets 8 consecutive k of column 16*(g%2) + i;
        // lanes 32..63 take the next 16 k, as the MFMA operand wants.
        const int g = lane >> 4, s = lane & 15;
        const int krow = 16 * (g >> 1) + (s >> 1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n = q * Cfg::WTN + nt * 32 + 16 * (g & 1) + 8 * (s & 1);
            b_rd[nt] = krow * B_ROW + (((n >> 4) ^ swz_b8(krow)) << 4) + (n & 15);
        }
    }
    // a_x: the lane's A address with the half-iteration's parity folded in
    // (bit 2 of the chunk index); stage_off: the B stage's byte offset
    auto read_a = [&](uint32_t slot_off, uint32_t a_x, int st, int mt) {
        const uint32_t x = (uint32_t)((st << 5) | ((mt & 1) << 6));
        return *(const u32x4 *)(lds + slot_off + mt * 4096 + (a_x ^ x));
    };
    // a slab (one MFMA step) is 16 k-rows of 16-bit B or 32 k-rows of int8
    auto read_b = [&](uint32_t stage_off, int st, int nt) {
        if constexpr (E == 2) {
            const uint8_t *base = lds + stage_off + b_rd[nt] + st * 16 * B_ROW;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(GSK_LDS(i16x4, base));
            const i16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16(GSK_LDS(i16x4, base + 4 * B_ROW));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            return u32x4{l2[0], l2[1], h2[0], h2[1]};
        } else {
            const uint8_t *base = lds + stage_off + b_rd[nt] + st * 32 * B_ROW;
            const s32x2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(GSK_LDS(s32x2, base));
            const s32x2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(GSK_LDS(s32x2, base + 8 * B_ROW));
            return u32x4{(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)hi[0], (uint32_t)hi[1]};
        }
    };

    f32x16 acc[MT][NT];
    u32x4 fa[2][MT], fb[2][NT];  // both 16-k slabs of one half-iteration

    WorkCursor cur = work_begin(P, p);
    WorkItem w;
    while (work_next(P, p, cur, w)) {
        int tm, tn;
        tile_coords(P, w.tile, &tm, &tn);
        const int m0 = tm * 256, n0 = tn * 256;
        const int k_lo = w.kb * BK;
        const int k_hi = w.ke * BK < args.K ? w.ke * BK : args.K;
        const int n = (k_hi - k_lo + HK - 1) / HK;  // half-iterations of this item (>= 1)
        // first k of the item's last slab (copy sources never start past it)
        const int kb_last = k_lo + ((k_hi - k_lo - 1) / HK) * HK;
        const int ka_last = k_lo + ((k_hi - k_lo - 1) / BK) * BK;

        // per-item source offsets (out of range: rows past M, columns past N);
        // group 0: off0 for rows 0-127, off1 for rows 128-255 (two named
        // arrays: one array indexed by the piece's parity was kept in scratch)
        uint32_t off0[4], off1[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (GRP == 0) {
                const int row = cp_row[j];
                off0[j] = m0 + row < args.M
                              ? (uint32_t)(row * args.lda * E + (cp_chunk[j] << 4))
                              : kOutOfRange;
                off1[j] = m0 + row + 128 < args.M
                              ? (uint32_t)((row + 128) * args.lda * E + (cp_chunk[j] << 4))
                              : kOutOfRange;
            } else {
                off0[j] = n0 + cp_chunk[j] * V < args.N
                              ? (uint32_t)(cp_row[j] * args.ldb * E + (cp_chunk[j] << 4))
                              : kOutOfRange;
                off1[j] = kOutOfRange;
            }
        }

        // Copy piece hc: group 0 the A row half (hc & 1) of iteration hc >> 1,
        // group 1 the B stage of half-iteration hc.  Pieces past the item's
        // end read nothing and zero their (free) buffer.
        auto copy_piece = [&](int hc) {
            if constexpr (GRP == 0) {
                const int ph = hc & 1;
                const int ka = k_lo + (hc >> 1) * BK;
                const bool whole = ka + BK <= k_hi;
                const int left = k_hi - ka;  // k values of this slab inside the item
                const uint8_t *src =
                    args.A + ((int64_t)m0 * args.lda + (ka <= ka_last ? ka : ka_last)) * E;
                const uint32_t dst = cp_lds + A_BASE + (uint32_t)(((hc >> 1) % SA) * A_SLOT) +
                                     (uint32_t)(ph * (A_SLOT / 2));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t off = ph ? off1[j] : off0[j];
                    copy16(rsrc_words(src), whole || cp_chunk[j] * V < left ? off : kOutOfRange,
                           dst + j * 4096);
                }
            } else {
                const int kb = k_lo + hc * HK;
                const bool whole = kb + HK <= k_hi;
                const int left = k_hi - kb;
                const uint8_t *src =
                    args.B + ((int64_t)(kb <= kb_last ? kb : kb_last) * args.ldb + n0) * E;
                const uint32_t dst = cp_lds + (uint32_t)((hc & (SB - 1)) * B_STAGE);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    copy16(rsrc_words(src),
                           whole || cp_row[j] < left ? off0[j] : kOutOfRange,
                           dst + j * 4096);
            }
        };
        // Fragments of half-iteration h: B stage h mod 4, A slot of iteration
        // h >> 1, A chunks 4..7 of the slab when h is odd
        auto read_frags = [&](int h) {
            const uint32_t slot_off = (uint32_t)(((h >> 1) % SA) * A_SLOT);
            const uint32_t stage_off = (uint32_t)((h & (SB - 1)) * B_STAGE);
            const uint32_t a_x = a_lane ^ ((uint32_t)(h & 1) << 6);
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    fa[st][mt] = read_a(slot_off, a_x, st, mt);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    fb[st][nt] = read_b(stage_off, st, nt);
            }
        };
        auto multiply = [&]() {
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int j = 0; j < MT * NT; ++j)
                    mfma_step<DT>(acc[j / NT][j % NT], fb[st][j % NT], fa[st][j / NT]);
        };
        // End of a phase: at most two copy batches of this wave in flight
        // (in-order completion), then the workgroup barrier; the scheduler
        // keeps everything on its side of it.
        auto phase_end = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<8>();
            barrier_only();
            __builtin_amdgcn_sched_barrier(0);
        };

#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[mt][nt] = f32x16{};

        // the previous item's copies are drained (below) and its LDS reads done
        barrier_only();
        copy_piece(0);
        copy_piece(1);
        copy_piece(2);
        phase_end();
        if constexpr (GRP == 0) {  // group 0 reads h = 0 and copies piece 3
            copy_piece(3);
            read_frags(0);
        }
        phase_end();

        // half-iteration h: phases 2h and 2h + 1
        for (int h = 0; h < n; ++h) {
            if constexpr (GRP == 0) {
                multiply();
                phase_end();
                if (h + 1 < n) {
                    copy_piece(h + 4);
                    read_frags(h + 1);
                }
                phase_end();
            } else {
                copy_piece(h + 3);
                read_frags(h);
                phase_end();
                multiply();
                phase_end();
            }
        }
        wait_vmcnt<0>();  // zero-fill copies past the end have landed

        finish_tile<256, 256, MT, NT, DT == 3>(acc, args, w, p, m0, n0, wave, lane,
                                               GRP * Cfg::WTM, q * Cfg::WTN);
    }
}

template <int DT>
__global__ __launch_bounds__(512, 1) void gemm_kernel_pp(KernelArgs args)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[PairTile<DT, 256, 256, 2, 4>::LDS];
    const int lane = threadIdx.x & 63;
    // wave index as a scalar: the group branch is uniform
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int p = logical_wg((int32_t)blockIdx.x, args.P.grid, args.P.xcds);
    if (wave < 4)
        gemm_pp_group<DT, 0>(args, lds, wave, lane, p);
    else
        gemm_pp_group<DT, 1>(args, lds, wave - 4, lane, p);
    if (args.split_fixup == 1)
        reduce_split_tiles<256, 256, 2, 4, DT == 3>(args, p, wave, lane);
}

template <int DT>
static int launch_gemm_pp(const KernelArgs &args, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_kernel_pp<DT>), dim3(grid), dim3(512), 0, stream, args);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <int DT, int BM, int BN, int WM, int WN>
static int launch_gemm(const KernelArgs &args, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, WM, WN>), dim3(grid),
                       dim3(Tile<DT, BM, BN, WM, WN>::NTH), 0, stream, args);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <int DT, int BM, int BN, int WM, int WN, bool STREAM>
static int launch_gemm_pair(const KernelArgs &args, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_kernel_pair<DT, BM, BN, WM, WN, STREAM>), dim3(grid),
                       dim3(PairTile<DT, BM, BN, WM, WN>::NTH), 0, stream, args);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Wave-specialised ping-pong kernel (fp16/bf16/int8, 256x256)
#define GSK_PP(DT)                                                                               \
    Variant{DT, 256, 256, PairTile<DT, 256, 256, 2, 4>::BK, 2, 4, 512,                          \
            (size_t)PairTile<DT, 256, 256, 2, 4>::LDS, 3, PairTile<DT, 256, 256, 2, 4>::SB,       \
            &launch_gemm_pp<DT>, (const void *)&gemm_kernel_pp<DT>,                              \
            &launch_fixup<256, 256, 2, 4, DT == 3>, 0}
// Register-staged kernel (fp32, int8 tiles the ping-pong kernel does not take, fp16/bf16 64x64)
#define GSK_STAGED(DT, BM, BN, WM, WN)                                                           \
    Variant{DT, BM, BN, Tile<DT, BM, BN, WM, WN>::BK, WM, WN, Tile<DT, BM, BN, WM, WN>::NTH,     \
            (size_t)Tile<DT, BM, BN, WM, WN>::LDS, 0, 0, &launch_gemm<DT, BM, BN, WM, WN>,        \
            (const void *)&gemm_kernel<DT, BM, BN, WM, WN>,                                      \
            &launch_fixup<BM, BN, WM, WN, DT == 3>, 0}
// Direct-to-LDS ring kernel with whole-row A copies (fp16/bf16)
#define GSK_PAIR_X(DT, BM, BN, WM, WN, ST)                                                       \
    Variant{DT, BM, BN, 64, WM, WN, PairTile<DT, BM, BN, WM, WN>::NTH,                           \
            (size_t)PairTile<DT, BM, BN, WM, WN>::LDS, 2, PairTile<DT, BM, BN, WM, WN>::SB,       \
            &launch_gemm_pair<DT, BM, BN, WM, WN, ST>,                                           \
            (const void *)&gemm_kernel_pair<DT, BM, BN, WM, WN, ST>,                             \
            &launch_fixup<BM, BN, WM, WN, false>, ST}
#define GSK_PAIR(DT, BM, BN, WM, WN) GSK_PAIR_X(DT, BM, BN, WM, WN, false)
// Non-temporal operand copies (GEMM_FLAG_STREAM_COPIES), for the layouts the
// long-K Stream-K shapes use
#define GSK_PAIR_STREAM(DT, BM, BN, WM, WN) GSK_PAIR_X(DT, BM, BN, WM, WN, true)

// The first entry matching a request wins, so each dtype's preferred kernel
// for a tile comes first.  Every entry is launched by the GPU tests (they walk
// this table through gemm_variant_info).
static const Variant kVariants[] = {
    // fp16 / bf16: direct-to-LDS ring kernel
    GSK_PAIR(1, 256, 256, 2, 4), GSK_PAIR(1, 256, 128, 4, 2), GSK_PAIR(1, 128, 256, 2, 4),
    GSK_PAIR(1, 128, 128, 2, 2),
    GSK_PAIR(2, 256, 256, 2, 4), GSK_PAIR(2, 256, 128, 4, 2), GSK_PAIR(2, 128, 256, 2, 4),
    GSK_PAIR(2, 128, 128, 2, 2),
    GSK_PAIR_STREAM(1, 256, 256, 2, 4), GSK_PAIR_STREAM(1, 256, 128, 4, 2),
    GSK_PAIR_STREAM(2, 256, 256, 2, 4), GSK_PAIR_STREAM(2, 256, 128, 4, 2),
    // fp16 / bf16 / int8: wave-specialised ping-pong kernel (256x256)
    GSK_PP(1), GSK_PP(2), GSK_PP(3),
    // fp16 / bf16 64x64 tiles (below the ring kernel's smallest tile), fp32, int8:
    // register-staged kernel
    GSK_STAGED(1, 64, 64, 2, 2), GSK_STAGED(2, 64, 64, 2, 2),
    GSK_STAGED(0, 128, 128, 2, 2), GSK_STAGED(0, 64, 64, 2, 2),
    GSK_STAGED(3, 256, 256, 4, 2), GSK_STAGED(3, 128, 128, 2, 2),
};

const Variant *variants(int *count)
{
    *count = (int)(sizeof(kVariants) / sizeof(kVariants[0]));
    return kVariants;
}

// ---------------------------------------------------------------- helpers

// dst (rows x ld_dst) = src (rows x cols, leading dimension ld_src), zero
// padded on the right; ld_dst * sizeof(T) is a multiple of 16 bytes and dst
// is 16-byte aligned.  One thread per 16-byte chunk of a destination row: a
// chunk that lies wholly inside the source row is one 16-byte load from the
// (only element-aligned) source address (gfx950 code objects run with
// unaligned global access enabled, and the compiler emits such loads itself
// for under-aligned data), a row's last, partial chunk is read element by
// element and zero padded, so no load reaches past its row.  Rows are
// strided over gridDim.y; no division.
constexpr int kPackThreads = 256;

template <typename T>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const T *__restrict__ src,
                                                            T *__restrict__ dst, int64_t rows,
                                                            int64_t cols, int64_t ld_src,
                                                            int64_t ld_dst)
{
    constexpr int V = 16 / (int)sizeof(T);  // elements per 16-byte chunk
    const int64_t c0 = ((int64_t)blockIdx.x * kPackThreads + threadIdx.x) * V;
    if (c0 >= ld_dst)
        return;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const T *s = src + r * ld_src + c0;
        u32x4 v;
        if (c0 + V <= cols) {
            __builtin_memcpy(&v, s, 16);
        } else {
            T e[V];
#pragma unroll
            for (int i = 0; i < V; ++i)
                e[i] = c0 + i < cols ? s[i] : T(0);
            __builtin_memcpy(&v, e, 16);
        }
        *(u32x4 *)(dst + r * ld_dst + c0) = v;
    }
}

template <typename T>
static void launch_pack_t(const void *src, void *dst, int64_t rows, int64_t cols, int64_t ld_src,
                          int64_t ld_dst, hipStream_t stream)
{
    constexpr int64_t PER = (int64_t)kPackThreads * (16 / sizeof(T));  // elements per workgroup
    const int64_t spans = (ld_dst + PER - 1) / PER;
    // enough rows per launch to keep every CU busy, each workgroup then loops
    const int64_t ys = rows < 32768 ? rows : 32768;
    hipLaunchKernelGGL(pack_kernel<T>, dim3((unsigned)spans, (unsigned)ys), dim3(kPackThreads), 0,
                       stream, (const T *)src, (T *)dst, rows, cols, ld_src, ld_dst);
}

int launch_pack(const void *src, void *dst, int64_t rows, int64_t cols, int64_t ld_src,
                int64_t ld_dst, int elem_size, hipStream_t stream)
{
    if (rows <= 0 || ld_dst <= 0)
        return 0;
    if (elem_size == 1)
        launch_pack_t<uint8_t>(src, dst, rows, cols, ld_src, ld_dst, stream);
    else if (elem_size == 2)
        launch_pack_t<uint16_t>(src, dst, rows, cols, ld_src, ld_dst, stream);
    else
        launch_pack_t<uint32_t>(src, dst, rows, cols, ld_src, ld_dst, stream);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Both operands' repacks in one launch, over one flat index of destination
// chunks: chunks [0, a.chunks) are A's, the rest B's.  A thread takes chunk
// k of its operand at row k / cpr, chunk k mod cpr, so every lane has work
// whatever the row length, where the row-per-workgroup kernel above leaves
// lanes idle on short rows and pays a workgroup per row.  The division is a
// multiply by a precomputed reciprocal: with s = ceil(log2 cpr), magic =
// ceil(2^(31+s) / cpr) and k < 2^31, (k * magic) >> (31 + s) equals k / cpr
// exactly (the rounding error of magic times k stays below 2^(31+s)).
// Chunk contents as in pack_kernel.
struct PackJob {
    const void *src;
    void *dst;
    int64_t ld_src, ld_dst;  // elements
    int64_t cols;            // elements of a source row
    uint64_t magic;          // ceil(2^shift / cpr)
    uint32_t shift;          // 31 + ceil(log2 cpr)
    uint32_t cpr;            // 16-byte chunks per destination row (ld_dst / V)
    uint32_t chunks;         // rows * cpr
};

template <typename T>
__global__ __launch_bounds__(kPackThreads) void pack_pair_kernel(PackJob a, PackJob b)
{
    constexpr int V = 16 / (int)sizeof(T);
    const uint32_t total = a.chunks + b.chunks;
    const uint32_t stride = gridDim.x * kPackThreads;
    for (uint32_t c = blockIdx.x * kPackThreads + threadIdx.x; c < total; c += stride) {
        const bool second = c >= a.chunks;
        const uint32_t k = second ? c - a.chunks : c;
        const uint32_t cpr = second ? b.cpr : a.cpr;
        const uint32_t r =
            (uint32_t)(((uint64_t)k * (second ? b.magic : a.magic)) >> (second ? b.shift : a.shift));
        const int64_t c0 = (int64_t)(k - r * cpr) * V;
        const int64_t cols = second ? b.cols : a.cols;
        const T *s = (const T *)(second ? b.src : a.src) + (int64_t)r * (second ? b.ld_src : a.ld_src) +
                     c0;
        T *d = (T *)(second ? b.dst : a.dst) + (int64_t)r * (second ? b.ld_dst : a.ld_dst) + c0;
        u32x4 v;
        if (c0 + V <= cols) {
            __builtin_memcpy(&v, s, 16);
        } else {
            T e[V];
#pragma unroll
            for (int i = 0; i < V; ++i)
                e[i] = c0 + i < cols ? s[i] : T(0);
            __builtin_memcpy(&v, e, 16);
        }
        *(u32x4 *)d = v;
    }
}

template <typename T>
static void launch_pack_pair_t(const PackJob &a, const PackJob &b, hipStream_t stream)
{
    const uint32_t total = a.chunks + b.chunks;
    // one chunk per thread: a thread that strides over several chunks has
    // only one load in flight at a time (each store waits for its load), so
    // a grid capped at a few workgroups per CU moved the large repacks ~7%
    // slower than one workgroup per 256 chunks (total < 2^31: < 2^23 blocks)
    const uint32_t blocks = (total + kPackThreads - 1) / kPackThreads;
    hipLaunchKernelGGL(pack_pair_kernel<T>, dim3(blocks), dim3(kPackThreads), 0, stream, a, b);
}

int launch_pack_pair(const void *a_src, void *a_dst, int64_t a_rows, int64_t a_cols,
                     int64_t a_ld_src, int64_t a_ld_dst, const void *b_src, void *b_dst,
                     int64_t b_rows, int64_t b_cols, int64_t b_ld_src, int64_t b_ld_dst,
                     int elem_size, hipStream_t stream)
{
    const int64_t V = 16 / elem_size;
    const int64_t a_chunks = a_rows > 0 ? a_rows * (a_ld_dst / V) : 0;
    const int64_t b_chunks = b_rows > 0 ? b_rows * (b_ld_dst / V) : 0;
    if (a_chunks + b_chunks == 0)
        return 0;
    if (a_chunks + b_chunks >= ((int64_t)1 << 31)) {
        // beyond the flat 32-bit chunk index: one row-per-workgroup launch each
        if (a_chunks && launch_pack(a_src, a_dst, a_rows, a_cols, a_ld_src, a_ld_dst, elem_size,
                                    stream))
            return -3;
        if (b_chunks && launch_pack(b_src, b_dst, b_rows, b_cols, b_ld_src, b_ld_dst, elem_size,
                                    stream))
            return -3;
        return 0;
    }
    auto job = [V](const void *src, void *dst, int64_t ld_src, int64_t ld_dst, int64_t cols,
                   int64_t chunks) {
        const uint32_t cpr = (uint32_t)(ld_dst / V > 0 ? ld_dst / V : 1);
        uint32_t s = 0;
        while (((uint64_t)1 << s) < cpr)
            ++s;
        const uint64_t shift = 31 + s;
        const uint64_t magic = (((uint64_t)1 << shift) + cpr - 1) / cpr;
        return PackJob{src, dst, ld_src, ld_dst, cols, magic, (uint32_t)shift, cpr,
                       (uint32_t)chunks};
    };
    const PackJob a = job(a_src, a_dst, a_ld_src, a_ld_dst, a_cols, a_chunks);
    const PackJob b = job(b_src, b_dst, b_ld_src, b_ld_dst, b_cols, b_chunks);
    if (elem_size == 1)
        launch_pack_pair_t<uint8_t>(a, b, stream);
    else if (elem_size == 2)
        launch_pack_pair_t<uint16_t>(a, b, stream);
    else
        launch_pack_pair_t<uint32_t>(a, b, stream);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <typename T>
__global__ void zero_kernel(T *__restrict__ C, int64_t count)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        C[i] = T(0);
}

int launch_zero(void *C, int64_t count, int elem_size, hipStream_t stream)
{
    if (count <= 0)
        return 0;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 8192)
        blocks = 8192;
    if (elem_size == 2)
        hipLaunchKernelGGL(zero_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (uint16_t *)C, count);
    else
        hipLaunchKernelGGL(zero_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (uint32_t *)C, count);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace gsk
