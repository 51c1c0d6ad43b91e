// Internal interface between the host API (api.hip) and the gfx950 kernels
// (kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "schedule.h"

namespace gsk {

// Everything one GEMM launch needs, passed by value as the kernel argument.
struct KernelArgs {
    const uint8_t *A;      // M x lda elements, row-major, 16-byte aligned rows
    const uint8_t *B;      // K x ldb elements, row-major, 16-byte aligned rows
    uint8_t *C;            // M x ldc elements of c_dtype
    int32_t c_dtype;       // 0: fp32 C; 1: fp16 C; 2: bf16 C (rounded to nearest even)
    float *partials;       // Stream-K partial tiles: bm*bn floats per slot
    int32_t *flags;        // one "partial ready" flag per slot (0 between runs)
    int32_t *counters;     // split fixup: readers done per split tile (0 between runs)
    int32_t *status;       // workspace status word (1 = a fixup wait gave up)
    int32_t split_fixup;   // 0: the head's workgroup adds every partial;
                           // 1: every piece is parked and the tile's workgroups
                           //    each reduce a share of its blocks;
                           // 2: every piece is parked, without flags, and a
                           //    second kernel reduces the split tiles
    int32_t M, N, K;
    int32_t lda, ldb, ldc; // leading dimensions in elements
    int32_t c_vec;         // 1: N % 4 == 0 and C 4-element aligned: vector stores in every
                           //    tile (otherwise only in tiles left of column N)
    int32_t spin_limit;    // polls before a fixup wait gives up
    int32_t drop_signal_wg;// testing: this workgroup never raises its piece's flag (-1: none)
    Partition P;
};

// One compiled GEMM kernel: input dtype and workgroup tile.
struct Variant {
    int dtype;             // gemm_dtype
    int bm, bn, bk;
    int wave_m, wave_n;    // wave grid of the workgroup
    int threads;
    size_t lds_bytes;
    int kind;              // 0: register-staged loads, 2: direct-to-LDS ring
    int stages;            // B stages of the kind-2 ring (0 for kind 0)
    int (*launch)(const KernelArgs &args, int grid, hipStream_t stream);
    const void *kernel;    // for occupancy queries
    // the two-kernel fixup's reduction kernel for this variant's piece layout
    int (*launch_fixup)(const KernelArgs &args, int grid, hipStream_t stream);
    int stream_copies;     // 1: operand copies carry the non-temporal hint
};

// All compiled variants; *count receives the number of entries.
const Variant *variants(int *count);

// Copy a rows x cols matrix of elem_size-byte elements with leading
// dimension ld_src into a dense rows x ld_dst buffer (ld_dst >= cols, a
// multiple of 16 bytes), zero-filling columns [cols, ld_dst).
int launch_pack(const void *src, void *dst, int64_t rows, int64_t cols, int64_t ld_src,
                int64_t ld_dst, int elem_size, hipStream_t stream);

// Both operands' repacks (as launch_pack) in one launch; an operand with
// rows = 0 is skipped.
int launch_pack_pair(const void *a_src, void *a_dst, int64_t a_rows, int64_t a_cols,
                     int64_t a_ld_src, int64_t a_ld_dst, const void *b_src, void *b_dst,
                     int64_t b_rows, int64_t b_cols, int64_t b_ld_src, int64_t b_ld_dst,
                     int elem_size, hipStream_t stream);

// C[0 .. count) = 0 for elements of elem_size bytes (the K = 0 product).
int launch_zero(void *C, int64_t count, int elem_size, hipStream_t stream);

}  // namespace gsk
