// gfx950 (CDNA4) GEMM kernels: C = A.B with fp32 accumulation, one kernel
// body for every schedule (data-parallel, persistent, Stream-K, hybrid).
//
// A workgroup of 4 waves computes a BM x BN output tile; each wave owns a
// (BM/2) x (BN/2) sub-tile built from 32x32 MFMA blocks.  One MAC iteration
// consumes a BK-deep slab of A (BM x BK) and B (BK x BN), where BK is 128
// bytes of input per row (64 fp16/bf16 or 32 fp32 values).  Slabs are staged
// global -> registers -> LDS with two LDS buffers, so the loads of slab k+1
// are in flight while slab k is multiplied, and one barrier per iteration
// separates the two ("double-buffering" in the persistent matmul post on the
// Hugging Face activity feed page).
//
// Both operands sit in LDS as rows of 128 bytes with the reduction index k
// contiguous (A: one row per output row m; B transposed on its way in: one
// row per output column n), so every MFMA operand is one 16-byte LDS read.
// The 16-byte chunks of a row are XOR-swizzled with (row ^ row >> 3) & 7:
// the 32 rows one fragment read touches, and the rows eight apart that one
// B write touches, land in distinct bank groups.
//
// The MFMA is issued with the operands swapped (B^T as the "A" operand), so
// the 32x32 accumulator block holds C^T: each lane then owns four consecutive
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

constexpr uint32_t kOutOfRange = 0x80000000u;
// Buffer descriptor word 3 for gfx9-family raw (untyped, stride 0) buffers.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff,
                                             kRsrcWord3);
}

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
    static constexpr int E = DT == 0 ? 4 : 2;         // bytes per element
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
    } else {
        // fp32: a lane's chunk is 4 consecutive k; instruction e takes element e
        // from both operands, so the same k meets the same k.
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, bt[e]),
                                                       __builtin_bit_cast(float, a[e]), acc, 0, 0,
                                                       0);
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
            compute_slab(s);
            store_slab(s ^ 1);
            __syncthreads();
            s ^= 1;
        }
        compute_slab(s);

        // Fragment f of this thread: block (mt, nt), row group g (4 rows of C^T,
        // i.e. 4 consecutive columns of C).
        if (w.role == ROLE_CONTRIB) {
            // Tail of a split tile: park it in this workgroup's slot, then signal.
            float *slot = args.partials + (int64_t)p * (BM * BN);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int f = ((wave * MT + mt) * NT + nt) * 4 + g;
                        *(f32x4 *)(slot + (f * 64 + lane) * 4) =
                            f32x4{acc[mt][nt][4 * g], acc[mt][nt][4 * g + 1],
                                  acc[mt][nt][4 * g + 2], acc[mt][nt][4 * g + 3]};
                    }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __syncthreads();
            if (tid == 0)
                __hip_atomic_store(args.flags + p, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            continue;
        }
        if (w.role == ROLE_OWNER) {
            // Head of a split tile: wait for every later workgroup on the tile,
            // then add their partials in ascending workgroup (= ascending k) order.
            if (tid == 0) {
                for (int q = p + 1; q <= w.peer_last; ++q) {
                    int spins = 0;
                    while (__hip_atomic_load(args.flags + q, __ATOMIC_ACQUIRE,
                                             __HIP_MEMORY_SCOPE_AGENT) == 0) {
                        if (++spins > args.spin_limit) {
                            __hip_atomic_store(args.status, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                    }
                    // Consumed: leave the flag clear for the next run.
                    __hip_atomic_store(args.flags + q, 0, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            __syncthreads();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            for (int q = p + 1; q <= w.peer_last; ++q) {
                const float *slot = args.partials + (int64_t)q * (BM * BN);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int f = ((wave * MT + mt) * NT + nt) * 4 + g;
                            f32x4 v = *(const f32x4 *)(slot + (f * 64 + lane) * 4);
                            acc[mt][nt][4 * g] += v[0];
                            acc[mt][nt][4 * g + 1] += v[1];
                            acc[mt][nt][4 * g + 2] += v[2];
                            acc[mt][nt][4 * g + 3] += v[3];
                        }
            }
        }

        // Store the tile: lane holds C[m][n .. n+3] for each fragment.
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = m0 + wy * Cfg::WTM + mt * 32 + l32;
            if (m >= args.M)
                continue;
            float *crow = args.C + (int64_t)m * args.ldc;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = n0 + wx * Cfg::WTN + nt * 32 + 8 * g + 4 * half;
                    f32x4 v = f32x4{acc[mt][nt][4 * g], acc[mt][nt][4 * g + 1],
                                    acc[mt][nt][4 * g + 2], acc[mt][nt][4 * g + 3]};
                    if (args.c_vec && n + 3 < args.N) {
                        *(f32x4 *)(crow + n) = v;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < args.N)
                                crow[n + e] = v[e];
                    }
                }
        }
    }
}

template <int DT, int BM, int BN, int WM, int WN>
static int launch_gemm(const KernelArgs &args, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, WM, WN>), dim3(grid),
                       dim3(Tile<DT, BM, BN, WM, WN>::NTH), 0, stream, args);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

#define GSK_VARIANT(DT, BM, BN, WM, WN)                                                          \
    Variant{DT, BM, BN, Tile<DT, BM, BN, WM, WN>::BK, Tile<DT, BM, BN, WM, WN>::NTH,             \
            (size_t)Tile<DT, BM, BN, WM, WN>::LDS, &launch_gemm<DT, BM, BN, WM, WN>,             \
            (const void *)&gemm_kernel<DT, BM, BN, WM, WN>}

static const Variant kVariants[] = {
    GSK_VARIANT(1, 256, 256, 2, 2), GSK_VARIANT(1, 256, 128, 2, 2),
    GSK_VARIANT(1, 128, 256, 2, 2), GSK_VARIANT(1, 128, 128, 2, 2),
    GSK_VARIANT(1, 64, 64, 2, 2),
    GSK_VARIANT(2, 256, 256, 2, 2), GSK_VARIANT(2, 256, 128, 2, 2),
    GSK_VARIANT(2, 128, 256, 2, 2), GSK_VARIANT(2, 128, 128, 2, 2),
    GSK_VARIANT(2, 64, 64, 2, 2),
    GSK_VARIANT(0, 128, 128, 2, 2), GSK_VARIANT(0, 64, 64, 2, 2),
};

const Variant *variants(int *count)
{
    *count = (int)(sizeof(kVariants) / sizeof(kVariants[0]));
    return kVariants;
}

// ---------------------------------------------------------------- helpers

// dst (rows x ld_dst) = src (rows x cols, leading dimension ld_src), zero
// padded on the right; one thread per destination element.
template <typename T>
__global__ void pack_kernel(const T *__restrict__ src, T *__restrict__ dst, int64_t rows,
                            int64_t cols, int64_t ld_src, int64_t ld_dst)
{
    const int64_t total = rows * ld_dst;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / ld_dst, c = i - (i / ld_dst) * ld_dst;
        dst[i] = c < cols ? src[r * ld_src + c] : T(0);
    }
}

int launch_pack(const void *src, void *dst, int64_t rows, int64_t cols, int64_t ld_src,
                int64_t ld_dst, int elem_size, hipStream_t stream)
{
    const int64_t total = rows * ld_dst;
    if (total <= 0)
        return 0;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192)
        blocks = 8192;
    if (elem_size == 2)
        hipLaunchKernelGGL(pack_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint16_t *)src, (uint16_t *)dst, rows, cols, ld_src, ld_dst);
    else
        hipLaunchKernelGGL(pack_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint32_t *)src, (uint32_t *)dst, rows, cols, ld_src, ld_dst);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

__global__ void zero_kernel(float *__restrict__ C, int64_t count)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        C[i] = 0.0f;
}

int launch_zero(float *C, int64_t count, hipStream_t stream)
{
    if (count <= 0)
        return 0;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 8192)
        blocks = 8192;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, C, count);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace gsk
