// Hardware ceilings of the MI355X paths the GEMM kernels lean on, measured
// by small in-bounds kernels (not part of the library; run by
// `python -m persistent_stream_tiling_amd.profiling ceilings`):
//
//   mfma     back-to-back v_mfma_f32_32x32x16_f16 on register operands, four
//            independent accumulators per wave, one or two waves per SIMD:
//            the matrix-core rate the power limit allows with no memory work;
//            with the same operands in every MFMA, or with four pseudo-random
//            operand pairs taken in turn (every MFMA's operands differ from
//            the previous one's, as in a GEMM); and v_mfma_i32_32x32x32_i8 on
//            pseudo-random bytes.
//   lds      16-byte LDS reads (ds_read_b128), 4..16 waves per CU.
//   copy     the 4096^3 fp16 GEMM's operand traffic: 256 workgroups of 8
//            waves, one 256x256 tile each, copying the A slab (256 rows x 128
//            bytes) and the B slab (64 rows x 512 bytes) of every 64-deep
//            iteration global -> LDS (buffer_load_dwordx4 ... lds), waiting
//            for each iteration's copies before the next; tiles dealt to the
//            dies in hardware order, in 4x8 blocks per die, or every
//            workgroup reading the same tile's panels (all L2 hits).
//   mix      the same copies plus, per wave and iteration, the 32 MFMAs a
//            128x64 wave tile of that GEMM issues, with no LDS fragment reads
//            (and the MFMAs alone).
//   reads    the 4096^3 GEMM's MFMAs plus its LDS fragment reads, with no
//            copies and no barriers: 256 workgroups, each wave running its
//            wave tile's 32x32x16 MFMAs over 256 16-deep slabs while it reads
//            the next slab's fragments between them (A: one ds_read_b128 per
//            32-row block; B: two transposing ds_read_b64_tr_b16 per 32-column
//            block).  Eight waves of 128x64 (the ping-pong kernel's wave tile,
//            8 reads per 8 MFMAs) against four waves of 128x128 (12 reads per
//            16 MFMAs, one wave per SIMD); then with a barrier per
//            half-iteration and with the operand copies (the ring kernel's
//            structure), and with zero or pseudo-random fragment values.
//
// Every launch is preceded by a 512 MiB fill that evicts L2 and the Infinity
// Cache; times are medians of 6 runs.  Every global and LDS offset stays
// inside its buffer (the copy offsets reach exactly the last byte of the
// 4096 x 4096 fp16 matrices); no kernel waits on another workgroup.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdio.h>
#include <stdlib.h>
#include <vector>

#define CHECK(x)                                                                              \
    do {                                                                                      \
        hipError_t e_ = (x);                                                                  \
        if (e_ != hipSuccess) {                                                               \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);    \
            exit(1);                                                                          \
        }                                                                                     \
    } while (0)

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kIters = 64;            // 64-deep iterations of a 4096-deep product
constexpr int kLd = 8192;             // bytes per row of a 4096-wide fp16 matrix
constexpr size_t kMat = 32u << 20;    // bytes of a 4096 x 4096 fp16 matrix

__device__ __forceinline__ i32x4 rsrc_words(const void *base)
{
    const uint64_t b = (uint64_t)base;
    return i32x4{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xffff), 0x7fffffff, 0x00020000};
}

// 16 bytes per lane from buffer offset voff into LDS at lds_addr + 16 * lane
__device__ __forceinline__ void copy16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc)
                 : "m0");
}

__global__ __launch_bounds__(256) void mfma_kernel(float *out, int iters, float seed)
{
    f32x16 acc[4] = {};
    f16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(seed * (float)(threadIdx.x + i));
        b[i] = (_Float16)(seed * (float)(i - 3));
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
    float s = 0.0f;
    for (int j = 0; j < 4; ++j)
        for (int e = 0; e < 16; ++e)
            s += acc[j][e];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef int s32x4 __attribute__((ext_vector_type(4)));
typedef int s32x16 __attribute__((ext_vector_type(16)));

// int8: back-to-back v_mfma_i32_32x32x32_i8 (32x32x32, int32 sums), eight
// independent accumulators per wave, pseudo-random operands (four pairs taken
// in turn, as in mfma_rand_kernel), one or two waves per SIMD
__global__ __launch_bounds__(256) void mfma_i8_kernel(int *out, int iters)
{
    s32x16 acc[8] = {};
    s32x4 a[4], b[4];
    for (int j = 0; j < 4; ++j)
        for (int e = 0; e < 4; ++e) {
            const uint32_t h = ((uint32_t)(threadIdx.x * 37 + j * 4 + e) + 1u) * 2654435761u;
            a[j][e] = (int)h;
            b[j][e] = (int)((h ^ (h >> 13)) * 2246822519u);
        }
    for (int it = 0; it < iters; it += 2)
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int j = u & 7, k = (u + (u >> 3)) & 3;
            acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[u & 3], b[k], acc[j], 0, 0, 0);
        }
    int s = 0;
    for (int j = 0; j < 8; ++j)
        for (int e = 0; e < 16; ++e)
            s += acc[j][e];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// An fp16 value from hash bits: sign and 10 mantissa bits from the hash,
// magnitude 1/8 .. 2.
__device__ __forceinline__ uint32_t probe_half(uint32_t h)
{
    return ((h >> 31) << 15) | ((12u + ((h >> 20) & 3u)) << 10) | (h & 0x3ffu);
}

// four operand pairs of pseudo-random fp16 values; MFMA u of a group of 16
// pairs A operand j = u % 4 with B operand (j + u / 4) % 4
__global__ __launch_bounds__(256) void mfma_rand_kernel(float *out, int iters)
{
    f32x16 acc[4] = {};
    u32x4 a[4], b[4];
    for (int j = 0; j < 4; ++j)
        for (int e = 0; e < 4; ++e) {
            const uint32_t h = ((uint32_t)(threadIdx.x * 37 + j * 4 + e) + 1u) * 2654435761u;
            const uint32_t h2 = (h ^ (h >> 13)) * 2246822519u;
            a[j][e] = probe_half(h) | (probe_half(h2) << 16);
            b[j][e] = probe_half(h2 ^ 0x5bd1e995u) | (probe_half(h * 3u) << 16);
        }
    for (int it = 0; it < iters; it += 4)
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int j = u & 3, k = (j + (u >> 2)) & 3;
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[j]),
                                                            __builtin_bit_cast(f16x8, b[k]),
                                                            acc[j], 0, 0, 0);
        }
    float s = 0.0f;
    for (int j = 0; j < 4; ++j)
        for (int e = 0; e < 16; ++e)
            s += acc[j][e];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void lds_kernel(uint32_t *out, int iters)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[64 * 1024];
    for (int i = threadIdx.x; i < 64 * 1024 / 4; i += blockDim.x)
        ((uint32_t *)lds)[i] = (uint32_t)i * 2654435761u;
    __syncthreads();
    u32x4 x = u32x4{0, 0, 0, 0};
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t base = (uint32_t)(wave * 16384 + lane * 16);
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < 16; ++j)
            x ^= *(const u32x4 *)(lds + ((base + j * 1024 + it * 64) & (64 * 1024 - 16)));
    out[blockIdx.x * blockDim.x + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

// order 0: hardware order (die = workgroup id mod 8), tiles row-major;
// order 1: die x holds a 4 x 8 block of tiles; order 2: all the same tile.
template <int NMFMA, bool COPY>
__global__ __launch_bounds__(512, 1) void copy_kernel(const uint8_t *A, const uint8_t *B,
                                                      int order, float *out)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[128 * 1024];
    const int hw = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int tm = 0, tn = 0;
    if (order == 0) {
        tm = hw / 16;
        tn = hw % 16;
    } else if (order == 1) {
        const int die = hw % 8, slot = hw / 8;
        tm = 4 * (die / 2) + slot / 8;
        tn = 8 * (die % 2) + slot % 8;
    }
    const uint8_t *a0 = A + (size_t)tm * 256 * kLd;
    const uint8_t *b0 = B + (size_t)tn * 512;
    const uint32_t lds_base =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds;
    uint32_t a_off[4], b_off[4];
    for (int j = 0; j < 4; ++j) {
        const int blk = j * 8 + wave;  // 1 KiB block of a 32 KiB slab
        a_off[j] = (uint32_t)((blk * 8 + (lane >> 3)) * kLd + (lane & 7) * 16);
        b_off[j] = (uint32_t)((blk * 2 + (lane >> 5)) * kLd + (lane & 31) * 16);
    }
    f32x16 acc[4] = {};
    f16x8 x, y;
    for (int i = 0; i < 8; ++i) {
        x[i] = (_Float16)(0.001f * (float)(lane + i));
        y[i] = (_Float16)(0.002f * (float)(i - 3));
    }
    for (int it = 0; it < kIters; ++it) {
        const i32x4 ra = rsrc_words(a0 + it * 128);
        const i32x4 rb = rsrc_words(b0 + (size_t)it * 64 * kLd);
        const uint32_t slot = lds_base + (uint32_t)((it & 1) * 65536 + wave * 1024);
        if (COPY) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                copy16(ra, a_off[j], slot + j * 8192);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                copy16(rb, b_off[j], slot + 32768 + j * 8192);
        }
#pragma unroll
        for (int m = 0; m < NMFMA; ++m)
            acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, acc[m & 3], 0, 0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    float s = 0.0f;
    for (int j = 0; j < 4; ++j)
        for (int e = 0; e < 16; ++e)
            s += acc[j][e];
    out[hw * 512 + threadIdx.x] = s;
}

#define PROBE_LDS(T, p) ((__attribute__((address_space(3))) T *)(p))

// MT x NT blocks of 32x32 per wave (MT = 4: 128 rows; NT = 2 or 4: 64 or 128
// columns).  The A fragments come from 128-byte rows at 64 KiB and the B
// fragments from 512-byte k-rows in two 8 KiB stages, both with the library
// kernels' XOR swizzles (A row r's chunk c at c ^ ((r ^ r >> 3) & 7); B k-row
// r's chunk c at c ^ {0, 6, 10, 12}[r & 3]).  Largest byte read: 64 KiB + 255 rows
// of 128 bytes + 3 blocks of 4 KiB + 127 = 110591 (A) and 11 k-rows of 512
// + 31 chunks of 16 + 14 + 8 KiB + 2 KiB + 8 = 16390 (B), inside the 160 KiB.
//
// BAR: a workgroup barrier once per 32-deep half-iteration, between its two
// slabs (where the ring kernel has its).  COPY (eight waves only): the
// 4096^3 operand copies of the copy probe (4x8 tile block per die) issued
// during the second slab's MFMAs, four per wave and half-iteration (the A
// slab of iteration h/2 on even h, its B slab on odd h), into a 32 KiB LDS
// region that no fragment read touches ([20480, 53248)); before the
// barrier point each wave waits until only the latest half-iteration's
// copies are in flight, as the ring kernel does.
//
// RAND: the fragments hold pseudo-random fp16 values (sign and 10 mantissa
// bits from a hash of the position, magnitude 1/8 .. 2) instead of zeros.
// The matrix cores' power, and with it the clock the power limit allows,
// depends on how many operand bits toggle: zero (or constant) operands run
// faster than a real product's.
template <int MT, int NT, bool BAR, bool COPY, bool RAND = false>
__global__ __launch_bounds__(64 * 8 * 2 / NT, 1) void reads_kernel(int slabs, const uint8_t *A,
                                                                   const uint8_t *B, float *out)
{
    static_assert(!COPY || NT == 2, "the copies are dealt to eight waves");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[160 * 1024];
    for (int i = threadIdx.x; i < 160 * 1024 / 4; i += blockDim.x) {
        const uint32_t h0 = ((uint32_t)i + blockIdx.x * 40960u) * 2654435761u;
        const uint32_t h1 = (h0 ^ (h0 >> 15)) * 2246822519u;
        ((uint32_t *)lds)[i] = RAND ? probe_half(h0) | (probe_half(h1) << 16) : 0u;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    const int row = ((wave >> 1) * 128 + l32) & 255;
    const uint32_t a_lane =
        65536u + (uint32_t)(row * 128) + (uint32_t)((half ^ ((row ^ (row >> 3)) & 7)) << 4);
    const int g = lane >> 4, si = lane & 15, krow = 8 * (g >> 1) + (si >> 2);
    uint32_t b_lane[NT];
    for (int nt = 0; nt < NT; ++nt) {
        const int n = ((wave & 3) * NT * 32 + nt * 32 + 16 * (g & 1) + 4 * (si & 3)) & 255;
        const int swz = (0xCA60 >> ((krow & 3) * 4)) & 0xF;
        b_lane[nt] = (uint32_t)(krow * 512 + ((((n >> 3) ^ swz) & 31) << 4) + (n & 7) * 2);
    }
    auto read_a = [&](int slab, int mt) {
        const uint32_t x = (uint32_t)(((slab & 1) << 5) | (((slab >> 1) & 1) << 6));
        return *(const u32x4 *)(lds + ((a_lane ^ x) + mt * 4096));
    };
    auto read_b = [&](int slab, int nt) {
        const uint8_t *p = lds + b_lane[nt] + (slab & 1) * 8192;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(PROBE_LDS(i16x4, p));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(PROBE_LDS(i16x4, p + 2048));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };
    // copy sources: the copy probe's order 1 (die x holds a 4 x 8 block of tiles)
    const int die = blockIdx.x % 8, slot = blockIdx.x / 8;
    const uint8_t *a0 = A + (size_t)(4 * (die / 2) + slot / 8) * 256 * kLd;
    const uint8_t *b0 = B + (size_t)(8 * (die % 2) + slot % 8) * 512;
    uint32_t a_off[4], b_off[4];
    for (int j = 0; j < 4; ++j) {
        const int blk = j * 8 + wave;
        a_off[j] = (uint32_t)((blk * 8 + (lane >> 3)) * kLd + (lane & 7) * 16);
        b_off[j] = (uint32_t)((blk * 2 + (lane >> 5)) * kLd + (lane & 31) * 16);
    }
    const uint32_t cp_lds =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds + 20480u +
        (uint32_t)wave * 1024u;
    f32x16 acc[MT][NT];
    for (int i = 0; i < MT; ++i)
        for (int j = 0; j < NT; ++j)
            acc[i][j] = f32x16{};
    u32x4 fa[2][MT], fb[2][NT];
    for (int mt = 0; mt < MT; ++mt)
        fa[0][mt] = read_a(0, mt);
    for (int nt = 0; nt < NT; ++nt)
        fb[0][nt] = read_b(0, nt);
    for (int s = 0; s < slabs; s += 2) {
        const int h = s >> 1, it = h >> 1;
        const i32x4 rsrc = (h & 1) ? rsrc_words(b0 + (size_t)it * 64 * kLd) : rsrc_words(a0 + it * 128);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (u == 1) {
                if (COPY)
                    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
                if (BAR)
                    __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
            // MFMAs on slab s + u, the fragments of slab s + u + 1 read between them
#pragma unroll
            for (int j = 0; j < MT * NT; ++j) {
                if (COPY && u == 1 && j >= MT * NT - 4) {
                    const int c = j - (MT * NT - 4);
                    // a bitwise select: a conditional here made the compiler keep
                    // both offset arrays in scratch memory
                    const uint32_t pick = 0u - (uint32_t)(h & 1);
                    copy16(rsrc, a_off[c] ^ ((a_off[c] ^ b_off[c]) & pick), cp_lds + c * 8192);
                }
                acc[j / NT][j % NT] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    __builtin_bit_cast(f16x8, fb[u][j % NT]), __builtin_bit_cast(f16x8, fa[u][j / NT]),
                    acc[j / NT][j % NT], 0, 0, 0);
                // in the order the next slab's MFMAs first need them
                if (j == 0)
                    fa[u ^ 1][0] = read_a(s + u + 1, 0);
                else if (j <= NT)
                    fb[u ^ 1][j - 1] = read_b(s + u + 1, j - 1);
                else if (j < MT + NT)
                    fa[u ^ 1][j - NT] = read_a(s + u + 1, j - NT);
                // keep this order: the reads a slab ahead of their MFMAs
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    float sum = 0.0f;
    for (int i = 0; i < MT; ++i)
        for (int j = 0; j < NT; ++j)
            for (int e = 0; e < 16; ++e)
                sum += acc[i][j][e];
    out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

struct Timer {
    hipEvent_t e0, e1;
    uint8_t *flush;
    Timer()
    {
        CHECK(hipEventCreate(&e0));
        CHECK(hipEventCreate(&e1));
        CHECK(hipMalloc(&flush, 512u << 20));
    }
    template <typename F>
    float median_us(F launch)
    {
        std::vector<float> t;
        for (int r = 0; r < 7; ++r) {
            CHECK(hipMemsetAsync(flush, r, 512u << 20));
            CHECK(hipEventRecord(e0));
            launch();
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(e1));
            CHECK(hipEventSynchronize(e1));
            float ms = 0.0f;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            if (r)
                t.push_back(ms * 1e3f);
        }
        std::sort(t.begin(), t.end());
        return t[t.size() / 2];
    }
};

int main()
{
    int cus = 0;
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    Timer T;
    float *fout;
    uint32_t *uout;
    uint8_t *A, *B;
    CHECK(hipMalloc(&fout, (size_t)cus * 8 * 512 * 4));
    CHECK(hipMalloc(&uout, (size_t)cus * 8 * 256 * 4));
    CHECK(hipMalloc(&A, kMat));
    CHECK(hipMalloc(&B, kMat));
    CHECK(hipMemset(A, 1, kMat));
    CHECK(hipMemset(B, 2, kMat));

    printf("| probe | configuration | us | rate |\n|---|---|---|---|\n");
    for (int wps : {1, 2}) {  // waves per SIMD: one or two workgroups of 4 waves per CU
        const int g = cus * wps, iters = 20000;
        const float us = T.median_us([&] {
            hipLaunchKernelGGL(mfma_kernel, dim3(g), dim3(256), 0, 0, fout, iters, 1e-3f);
        });
        const double flops = (double)g * 4 * iters * 4 * 32768.0;
        printf("| mfma | %d wave(s) per SIMD, %d x 4 MFMA 32x32x16 f16 per wave | %.1f | %.1f "
               "TFLOP/s (%.1f%% of 2516.6) |\n",
               wps, iters, us, flops / us / 1e6, flops / us / 1e6 / 2516.6 * 100);
    }
    for (int wps : {1, 2}) {
        const int g = cus * wps, iters = 20000;
        const float us = T.median_us([&] {
            hipLaunchKernelGGL(mfma_rand_kernel, dim3(g), dim3(256), 0, 0, fout, iters);
        });
        const double flops = (double)g * 4 * iters * 4 * 32768.0;
        printf("| mfma | %d wave(s) per SIMD, %d x 4 MFMA 32x32x16 f16 per wave, pseudo-random "
               "operands | %.1f | %.1f TFLOP/s (%.1f%% of 2516.6) |\n",
               wps, iters, us, flops / us / 1e6, flops / us / 1e6 / 2516.6 * 100);
    }
    for (int wps : {1, 2}) {
        const int g = cus * wps, iters = 20000;
        const float us = T.median_us([&] {
            hipLaunchKernelGGL(mfma_i8_kernel, dim3(g), dim3(256), 0, 0, (int *)fout, iters);
        });
        const double ops = (double)g * 4 * iters * 8 * 65536.0;
        printf("| mfma | %d wave(s) per SIMD, %d x 8 MFMA 32x32x32 i8 per wave, pseudo-random "
               "operands | %.1f | %.1f TOP/s (%.1f%% of 5033.2) |\n",
               wps, iters, us, ops / us / 1e6, ops / us / 1e6 / 5033.2 * 100);
    }
    for (int wpc : {1, 2, 4}) {  // workgroups of 4 waves per CU
        const int g = cus * wpc, iters = 20000;
        const float us = T.median_us(
            [&] { hipLaunchKernelGGL(lds_kernel, dim3(g), dim3(256), 0, 0, uout, iters); });
        const double bytes = (double)g * 256 * iters * 16 * 16.0;
        printf("| lds | %d workgroup(s) of 4 waves per CU, ds_read_b128 | %.1f | %.1f TB/s, %.0f "
               "B/clk/CU at 2.4 GHz |\n",
               wpc, us, bytes / us / 1e6, bytes / (us * 1e-6) / cus / 2.4e9);
    }
    const double copy_bytes = 256.0 * kIters * 65536;
    const char *orders[3] = {"hardware die order", "4x8 tile block per die", "one tile's panels (L2 hits)"};
    for (int order = 0; order < 3; ++order) {
        const float us = T.median_us([&] {
            hipLaunchKernelGGL((copy_kernel<0, true>), dim3(256), dim3(512), 0, 0, A, B, order, fout);
        });
        printf("| copy | 4096^3 operand slabs global -> LDS, %s | %.1f | %.2f TB/s, %.1f GB/s "
               "per CU |\n",
               orders[order], us, copy_bytes / us / 1e6, copy_bytes / us / 1e3 / 256);
    }
    const float m0 = T.median_us([&] {
        hipLaunchKernelGGL((copy_kernel<32, false>), dim3(256), dim3(512), 0, 0, A, B, 1, fout);
    });
    printf("| mix | no copies, 32 MFMAs per wave and iteration (the 4096^3 GEMM's MFMA work) | "
           "%.1f | %.0f TFLOP/s |\n",
           m0, 2.0 * 4096.0 * 4096.0 * 4096.0 / m0 / 1e6);
    const float m32 = T.median_us([&] {
        hipLaunchKernelGGL((copy_kernel<32, true>), dim3(256), dim3(512), 0, 0, A, B, 1, fout);
    });
    printf("| mix | the copies above (4x8 block per die) plus 32 MFMAs per wave and iteration "
           "(the 4096^3 GEMM's MFMA work) | %.1f | %.0f TFLOP/s-equivalent |\n",
           m32, 2.0 * 4096.0 * 4096.0 * 4096.0 / m32 / 1e6);
    auto reads_row = [&](const char *what, float us) {
        printf("| reads | %s | %.1f | %.0f TFLOP/s-equivalent |\n", what, us,
               2.0 * 4096.0 * 4096.0 * 4096.0 / us / 1e6);
    };
    reads_row("8 waves of 128x64: the 4096^3 GEMM's MFMAs and LDS fragment reads, no copies, "
              "no barriers",
              T.median_us([&] {
                  hipLaunchKernelGGL((reads_kernel<4, 2, false, false>), dim3(256), dim3(512), 0,
                                     0, 256, A, B, fout);
              }));
    reads_row("4 waves of 128x128 (one per SIMD): the same work", T.median_us([&] {
                  hipLaunchKernelGGL((reads_kernel<4, 4, false, false>), dim3(256), dim3(256), 0,
                                     0, 256, A, B, fout);
              }));
    reads_row("8 waves of 128x64, a barrier per half-iteration", T.median_us([&] {
                  hipLaunchKernelGGL((reads_kernel<4, 2, true, false>), dim3(256), dim3(512), 0,
                                     0, 256, A, B, fout);
              }));
    reads_row("8 waves of 128x64 plus the operand copies, no barriers", T.median_us([&] {
                  hipLaunchKernelGGL((reads_kernel<4, 2, false, true>), dim3(256), dim3(512), 0,
                                     0, 256, A, B, fout);
              }));
    reads_row("8 waves of 128x64 plus the operand copies and a barrier per half-iteration "
              "(the ring kernel's structure)",
              T.median_us([&] {
                  hipLaunchKernelGGL((reads_kernel<4, 2, true, true>), dim3(256), dim3(512), 0,
                                     0, 256, A, B, fout);
              }));
    reads_row("8 waves of 128x64, no copies, no barriers, pseudo-random fp16 fragments",
              T.median_us([&] {
                  hipLaunchKernelGGL((reads_kernel<4, 2, false, false, true>), dim3(256),
                                     dim3(512), 0, 0, 256, A, B, fout);
              }));
    reads_row("4 waves of 128x128 (one per SIMD), no copies, no barriers, pseudo-random fp16 "
              "fragments",
              T.median_us([&] {
                  hipLaunchKernelGGL((reads_kernel<4, 4, false, false, true>), dim3(256),
                                     dim3(256), 0, 0, 256, A, B, fout);
              }));
    reads_row("the ring kernel's structure (copies, barriers) with pseudo-random fp16 fragments",
              T.median_us([&] {
                  hipLaunchKernelGGL((reads_kernel<4, 2, true, true, true>), dim3(256),
                                     dim3(512), 0, 0, 256, A, B, fout);
              }));
    return 0;
}
