/*
 * gemm_sk -- tiled dense C = A.B on one MI355X (gfx950) with four work
 * schedules: data-parallel tiles, a persistent grid, Stream-K, and the
 * Stream-K + data-parallel hybrid.
 *
 * The operation.  C[i][j] = sum_k A[i][k] * B[k][j] for an M x K matrix A and
 * a K x N matrix B ("naive vs persistent matmul" post on the Hugging Face
 * activity feed page: the MxK . KxN product, computed one output tile at a
 * time as a sum-reduction across K).  A and B are fp32, fp16 or bf16; the
 * products are accumulated in fp32 (Triton issue #1393 "Stream-k matmul
 * implementation very slow...", final revision, where the accumulator type is
 * fp32 for fp16/bf16/fp32 inputs) and C is written as fp32 (or, with
 * GEMM_FLAG_C_INPUT_DTYPE, in the input dtype, as on that page).
 *
 * The schedules (same two pages):
 *   GEMM_DP          one workgroup per output tile; the hardware hands CUs new
 *                    workgroups as old ones finish (the post's "naive" matmul).
 *   GEMM_PERSISTENT  g workgroups (default: one per CU) stay alive and loop over
 *                    tiles p, p+g, p+2g, ... (the post's persistent matmul).
 *   GEMM_STREAMK     the T * ipt MAC iterations of all tiles are split evenly
 *                    over g workgroups, workgroup p getting iterations
 *                    [p*q + min(p,r), (p+1)*q + min(p+1,r)) with q = I / g and
 *                    r = I mod g (issue #1393, the first-wave kernel).  A tile
 *                    shared by several workgroups is finished by a fixup.
 *   GEMM_HYBRID      Stream-K over the first T_sk tiles, data-parallel over the
 *                    rest, with T_sk = T mod g, plus g more when two_tiles is on
 *                    and more than g tiles would remain (issue #1393, the host
 *                    wrapper of the final revision).
 *
 * Fixup (replaces the pages' lock + float atomic_add).  Of the workgroups that
 * share a split tile, the one covering the tile's first k-iteration (the
 * "owner") waits for the others, which each store their fp32 partial tile in
 * a workspace slot and raise a flag; the owner adds the partials to its own
 * accumulator one by one in ascending workgroup order (= ascending k) and
 * writes C.  For tiles cut into many pieces the same sums can instead be
 * spread over all of the tile's workgroups (GEMM_FLAG_FIXUP_SPLIT).  There are
 * no floating-point atomics, so one plan gives bitwise identical C on every
 * run.  Different schedules may differ in the last bits.
 *
 * Layout.  A is M x K row-major (leading dimension K), B is K x N row-major
 * (leading dimension N), C is M x N row-major (leading dimension N), fp32 or,
 * with GEMM_FLAG_C_INPUT_DTYPE, fp16/bf16.  A, B and C are device pointers; A
 * and B must be 16-byte aligned, C aligned to its element size.  C is fully
 * overwritten (no zero fill needed).  Rows whose byte length is not a multiple
 * of 16 are repacked into the workspace before the multiply.
 *
 * Threading.  Plans are immutable after creation and may be shared between
 * host threads.  gemm_last_error() is thread-local.
 */
#ifndef GEMM_SK_H
#define GEMM_SK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input dtype.  fp32/fp16/bf16 accumulate in fp32 and write fp32 C (or the
 * input dtype, GEMM_FLAG_C_INPUT_DTYPE).  GEMM_I8: int8 inputs accumulate in
 * int32, exactly, and C is int32 (the accumulator type issue #1393's final
 * revision picks for int8); K must stay below 2^17 so no sum can overflow. */
typedef enum { GEMM_F32 = 0, GEMM_F16 = 1, GEMM_BF16 = 2, GEMM_I8 = 3 } gemm_dtype;

typedef enum {
    GEMM_DP = 0,
    GEMM_PERSISTENT = 1,
    GEMM_STREAMK = 2,
    GEMM_HYBRID = 3
} gemm_schedule;

/* gemm_tiles.flags */
enum {
    /* Hybrid: use one-tile Stream-K (T_sk = T mod g) instead of the default
     * two-tile form (issue #1393, final revision's two_tiles switch). */
    GEMM_FLAG_ONE_TILE = 1u << 0,
    /* Do not remap workgroup ids so that each XCD gets a contiguous run of
     * tiles (for measuring what the remap buys). */
    GEMM_FLAG_NO_XCD_REMAP = 1u << 1,
    /* Bits 2 and 5 are reserved (they selected kernel families that are no
     * longer built); gemm_plan_create refuses a plan that sets them. */
    /* Stream-K fixup mode (default: split whenever some tile is cut):
     *  HEAD  the workgroup holding a split tile's k = 0 adds the other pieces
     *        one by one and stores the tile;
     *  SPLIT every piece is parked in the workspace; after their MAC work the
     *        tile's workgroups each add up and store a share of its blocks.
     *        A workgroup then walks its range as whole tiles, head piece, tail
     *        piece, so that workgroups running side by side read the same k
     *        range of A and B at the same time.
     * Both add the pieces of every element in ascending k order, so they give
     * identical bits. */
    GEMM_FLAG_FIXUP_HEAD = 1u << 3,
    GEMM_FLAG_FIXUP_SPLIT = 1u << 4,
    /* C is written in the input dtype instead of fp32: each fp32 sum is
     * rounded to the nearest fp16 / bf16 value (ties to even) as it is
     * stored.  This is the pages' output type: issue #1393's final revision
     * allocates C in A's dtype and casts the fp32 accumulator to it when it
     * stores a tile.  Stream-K partial tiles stay fp32 in the workspace and
     * only the finished sum is rounded, so the half-precision C of a plan is
     * exactly the rounding of the fp32 C of the same plan without this flag.
     * A no-op for fp32 inputs. */
    GEMM_FLAG_C_INPUT_DTYPE = 1u << 6,
    /* Testing the fixup's failure detection only: the highest-numbered
     * workgroup that parks a Stream-K piece never raises its flag, and every
     * fixup wait gives up after a few thousand polls (a few milliseconds)
     * instead of about a second.  A run of such a plan ends normally with
     * workspace status 1 (see gemm_workspace_status) and an invalid C.
     * gemm_plan_create refuses it for a plan that splits no tile. */
    GEMM_FLAG_DEBUG_DROP_SIGNAL = 1u << 7,
    /* Two-kernel Stream-K fixup: every piece of a split tile is parked in the
     * workspace without a flag, and a second kernel, launched by gemm_run on
     * the same stream, reduces each split tile in ascending k order (the same
     * additions, so the same bits, as the split fixup).  Nothing waits on
     * another workgroup, so the Stream-K grid may exceed the number of
     * workgroups that can be resident at once (e.g. two per CU, which issue
     * #1393 also tries). */
    GEMM_FLAG_FIXUP_TWO_KERNEL = 1u << 8,
    /* fp16/bf16 ring kernel: the operand copies carry the non-temporal cache
     * hint, so A and B lines are not kept for reuse.  Faster where each line
     * is read by few workgroups at a time (few tiles and a long K, e.g.
     * 512x512x65536 under Stream-K), slower where tiles share operand panels
     * in L2.  Built for 256x256 (2x4 waves) and 256x128 (4x2) tiles; other
     * tiles with this flag have no kernel. */
    GEMM_FLAG_STREAM_COPIES = 1u << 9,
    /* Tile order along a Hilbert curve over the tile grid instead of
     * GROUP_M bands (the "Inside NVIDIA GPUs: Anatomy of high performance
     * matmul kernels" page lists Hilbert curves among tile scheduling
     * policies): tile ids follow the classic curve on the power-of-two square
     * enclosing the grid, counting only tiles inside the grid, so runs of
     * consecutive ids (what one die and one wave of workgroups hold) cover
     * compact blocks of tiles on any grid shape.  group_m is ignored. */
    GEMM_FLAG_HILBERT_ORDER = 1u << 10,
    /* fp16/bf16/int8, 256x256 tiles: the wave-specialised ping-pong kernel
     * (kernel_kind 3), the default wherever it is built (256x256 tiles in
     * the 2x4 wave layout, without GEMM_FLAG_STREAM_COPIES); this flag asks
     * for it explicitly and refuses tiles without it.  Its eight waves form
     * two groups, one wave of each on every SIMD, that take turns: one group
     * runs a burst of MFMAs on fragments already in registers while the other
     * issues its share of the global -> LDS copies and reads its next
     * fragments ("naive vs persistent matmul" post on the Hugging Face
     * activity feed page: warp specialization and ping-pong scheduling, there
     * for NVIDIA's warp groups).  Same results as the ring kernel with the
     * same tile (the same MFMAs in the same order per element). */
    GEMM_FLAG_PING_PONG = 1u << 11,
    /* Never the ping-pong kernel: fp16/bf16 256x256 tiles then run the ring
     * kernel (kernel_kind 2), which is otherwise the default for the other
     * fp16/bf16 tiles (for comparing the two); int8 256x256 tiles run the
     * register-staged kernel (there is no int8 ring kernel). */
    GEMM_FLAG_RING_KERNEL = 1u << 12,
    /* Stream-K / hybrid: cut each of the T_sk Stream-K tiles into
     * s = min(floor(g / T_sk), ipt) pieces, one per workgroup, by the same
     * even-split rule Stream-K applies to the whole range (pieces of
     * floor(ipt/s) or ceil(ipt/s) iterations), instead of splitting all
     * T_sk * ipt iterations evenly over the g workgroups.  No workgroup's
     * range then crosses a tile boundary (a workgroup that runs pieces of two
     * tiles pays a second pipeline fill and a second parked piece, and both
     * tiles' fixups wait for it); workgroups p >= s * T_sk get no Stream-K
     * work.  With g = s * T_sk and s dividing ipt this is the pages' own split
     * (a fixed split-K).  Not on the pages.  Needs g >= T_sk. */
    GEMM_FLAG_TILE_SPLIT = 1u << 13
};

/* Tile and schedule knobs.  Every field 0 means "default". */
typedef struct {
    int32_t bm, bn;   /* output tile (multiples of 32 from the supported set;
                         default per dtype and shape) */
    int32_t bk;       /* k-depth of one MAC iteration, fixed per kernel: 64
                         for fp16/bf16, 32 for fp32, 128 for int8; 0 = any */
    int32_t grid;     /* g: workgroups of the persistent / Stream-K launch;
                         0 = number of CUs (issue #1393 uses the SM count).
                         fp16/bf16 Stream-K and hybrid with bm = bn = 0 and
                         grid = 0 (and no wave layout, stages or kernel
                         flag): the planner picks the tile (256x256,
                         256x128, 128x128, or 64x64 where that gives at
                         most one tile per CU) and g from a cost model fitted
                         on MI355X, among g = s*T that cut every tile into
                         s equal pieces (s in 1, 2, 3, 4, 6, 8, 16 dividing
                         the iterations per tile, g <= CUs) and g = CUs;
                         where every tile shape gives more than CUs tiles,
                         g = CUs, and the hybrid keeps one Stream-K wave
                         (T_sk = T mod g, as with GEMM_FLAG_ONE_TILE) and
                         cuts each of its Stream-K tiles into its own pieces
                         (as GEMM_FLAG_TILE_SPLIT).  (Issue #1393's
                         benchmark picks g per shape from a sweep; a library
                         call cannot.) */
    int32_t group_m;  /* tile-order group height (issue #1393 GROUP_M);
                         0 = 8, < 0 = plain row-major tile order (see also
                         GEMM_FLAG_HILBERT_ORDER) */
    uint32_t flags;   /* GEMM_FLAG_* */
    int32_t wave_m, wave_n; /* waves per workgroup along M and N (each wave
                               computes a (bm/wave_m) x (bn/wave_n) block);
                               0 = the default layout for the tile */
    int32_t stages;   /* B stages of the fp16/bf16 ring kernel (4); 0 = default */
} gemm_tiles;

/* Device description for planning without touching a GPU (host tests). */
typedef struct {
    int32_t cus;       /* compute units, e.g. 256 on MI355X */
    int32_t xcds;      /* dies that workgroups are dealt to in turn, e.g. 8 */
    int32_t wg_per_cu; /* co-resident workgroups of the chosen kernel per CU;
                          0 = 1 */
} gemm_device_desc;

typedef struct gemm_plan gemm_plan;

/*
 * Create a plan for C = A.B with the given shape, input dtype and schedule.
 * This is the host half of the final revision's wrapper (`matmul._call`) on
 * the Triton issue #1393 page: from M, N, K and the block shape it derives
 * the tile grid (tiles_m, tiles_n, T), the MAC iterations per tile
 * (ipt = ceil(K / bk)), the number of Stream-K tiles (the hybrid's T_sk) and
 * the per-workgroup share q, r of their iterations; here the result is kept
 * in an immutable plan instead of being recomputed on every call.
 *
 * tiles may be NULL (all defaults).  The device is the current HIP device.
 * M, N, K >= 0 (M or N = 0: nothing to do; K = 0: C is zero-filled).
 * Returns NULL on error (message in gemm_last_error()): negative sizes; a
 * matrix too large for the kernels' 32-bit offsets (M, N, K < 2^30, and one
 * tile's rows of A, C and one iteration's rows of B below 2^30 bytes, e.g.
 * N < 2^20 for 256-row tiles with fp32 C); an unknown dtype or schedule; a
 * reserved flag; an unsupported tile; or a Stream-K / hybrid grid larger than
 * the number of workgroups that can be resident at once (the in-kernel fixups
 * wait on other workgroups, so all of them must be running together; not
 * with GEMM_FLAG_FIXUP_TWO_KERNEL).
 */
gemm_plan *gemm_plan_create(int64_t M, int64_t N, int64_t K, gemm_dtype dtype,
                            gemm_schedule schedule, const gemm_tiles *tiles);

/* Same, for an explicit device description; needs no GPU.  A plan made this
 * way can be inspected but gemm_run refuses it unless its description matches
 * the current device. */
gemm_plan *gemm_plan_create_for_device(int64_t M, int64_t N, int64_t K, gemm_dtype dtype,
                                       gemm_schedule schedule, const gemm_tiles *tiles,
                                       const gemm_device_desc *device);

/*
 * Enqueue C = A.B on stream (a hipStream_t; NULL = the default stream).
 * This is the launch half of the same wrapper on the Triton issue #1393 page
 * (its first-wave Stream-K kernel, then its data-parallel kernel over the
 * remaining tiles); here one persistent launch runs both phases, plus a short
 * second launch for GEMM_FLAG_FIXUP_TWO_KERNEL plans and, for rows that are
 * not a multiple of 16 bytes, a repack of A and/or B into the workspace
 * before it.
 *
 * Asynchronous: never allocates, never synchronizes.  workspace is a device
 * buffer of at least gemm_plan_workspace_size(plan) bytes, 256-byte aligned,
 * zero-filled once when allocated; it may be NULL when that size is 0.  A run
 * leaves the workspace's flags zero again, so it can be reused by later runs
 * without clearing.  Two runs that overlap in time must not share a
 * workspace.  C points to M x N fp32 values, to fp16/bf16 values when the
 * plan was made with GEMM_FLAG_C_INPUT_DTYPE, or to int32 values for int8
 * inputs.  The caller owns A, B, C and the workspace.
 *
 * Co-residency.  Under Stream-K and hybrid plans that split a tile (and not
 * GEMM_FLAG_FIXUP_TWO_KERNEL), workgroups wait for pieces parked by other
 * workgroups of the same launch, which needs all g workgroups resident at
 * once.  The planner caps g at the device's resident capacity for this
 * kernel, but kernels running concurrently on other streams can hold CUs and
 * break that assumption.  The waits are bounded (about a second), so the
 * kernel always ends; a wait that gives up sets the workspace status word,
 * which gemm_workspace_status reads.  gemm_run cannot return that outcome
 * (it returns before the kernel runs): a caller that cannot rule out such a
 * wait must read the status after the run and treat a nonzero status as a
 * failed product (the Python binding does this by default).
 *
 * Returns 0, or -1 invalid argument (NULL or misaligned pointer), -2
 * workspace missing, -3 HIP launch error, -5 plan made for another device.
 */
int gemm_run(const gemm_plan *plan, const void *A, const void *B, void *C, void *workspace,
             void *stream);

/* Most workspace gemm_run_noalloc can provide: 80 MiB per device, held from
 * its first call on a device until the process ends.  That covers every
 * Stream-K / hybrid plan with tiles up to 256x128 at the default grid of 256
 * workgroups (64 MiB of partial slots in split mode), and 256x256 tiles up to
 * g = 160; plans whose operands are repacked also need room for the packed
 * copies. */
#define GEMM_NOALLOC_MAX_WORKSPACE ((size_t)80 << 20)

/*
 * gemm_run without a caller-owned workspace, for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * and harnesses that forbid hipMalloc.  It allocates nothing: the workspace is
 * a fixed array in the library's device memory (GEMM_NOALLOC_MAX_WORKSPACE
 * bytes per device, set up on the first call on each device).  The caller
 * passes A, B, C and the stream exactly as for gemm_run, and gets the same
 * bits as gemm_run with the same plan.
 *
 * Every call on a device shares that device's array, which keeps what the
 * last call left; each call clears the parts that must start at zero (status
 * word, flags, counters) with a fill kernel on the stream before the GEMM, so
 * an earlier call, even one whose fixup wait gave up, leaves no stale state.
 * Calls that overlap in time on one device race on the array: serialise them
 * (e.g. issue them on one stream).  gemm_workspace_status(plan, NULL, stream,
 * &status) reads the array's status word after a call.
 *
 * Returns what gemm_run returns, and -2 when the plan needs more workspace
 * than the array holds (message in gemm_last_error()).
 */
int gemm_run_noalloc(const gemm_plan *plan, const void *A, const void *B, void *C, void *stream);

/* Free a plan (NULL is ignored). */
void gemm_plan_destroy(gemm_plan *plan);

/* Bytes of workspace gemm_run needs (0 when none). */
size_t gemm_plan_workspace_size(const gemm_plan *plan);

/* Human-readable plan summary (tile grid, partition, launch) into buf; the
 * analogue of the debug print in the Triton issue #1393 final revision's
 * wrapper (M, N, K, block shape, tile counts, iterations per tile, Stream-K
 * tiles and the per-workgroup split).  Returns the length it needed (like
 * snprintf), or -1 on a NULL plan. */
int gemm_plan_describe(const gemm_plan *plan, char *buf, size_t len);

/* Message of the last failed call on this host thread ("" if none). */
const char *gemm_last_error(void);

/* ---- introspection (host only; used by the tests and the benchmark) ---- */

typedef struct {
    int64_t M, N, K;
    int32_t dtype, schedule;
    int32_t bm, bn, bk, group_m;
    uint32_t flags;
    int32_t wave_m, wave_n;
    int32_t kernel_kind;  /* 0 register-staged, 2 direct-to-LDS ring, 3 ping-pong */
    int32_t stages;
    int32_t split_fixup;  /* 1 when the Stream-K fixup is split (see flags) */
    int32_t max_pieces;   /* most workgroups sharing one Stream-K tile */
    int32_t tiles_m, tiles_n;
    int32_t tiles;        /* T */
    int32_t iters_per_tile; /* ipt = ceil(K / bk) */
    int32_t tiles_sk;     /* T_sk: tiles [0, T_sk) are split by Stream-K */
    int32_t tiles_dp;     /* T - T_sk */
    int64_t iters_sk;     /* T_sk * ipt */
    int32_t q, r;         /* iters_sk = q * g + r; with GEMM_FLAG_TILE_SPLIT
                             ipt = q * pieces_per_tile + r */
    int32_t g;            /* Stream-K / persistent workgroup count */
    int32_t launch_grid;  /* workgroups launched */
    int32_t threads;      /* threads per workgroup */
    int32_t cus, xcds, wg_capacity;
    int32_t pack_a, pack_b; /* operand repacked into the workspace */
    size_t workspace;
    size_t lds_bytes;
    int32_t pieces_per_tile; /* GEMM_FLAG_TILE_SPLIT: s (each Stream-K tile cut
                                into s pieces); 0 otherwise */
} gemm_plan_info;

int gemm_plan_get_info(const gemm_plan *plan, gemm_plan_info *out);

enum { GEMM_ROLE_FULL = 0, GEMM_ROLE_CONTRIB = 1, GEMM_ROLE_OWNER = 2 };

/* One unit of work of a workgroup: MAC iterations [k_begin, k_end) of a tile.
 * FULL: the whole tile, stored to C.  CONTRIB: a tail of a split tile, stored
 * to this workgroup's workspace slot.  OWNER: the head (k_begin = 0) of a split
 * tile, finished with the partials of workgroups wg+1 .. peer_last. */
typedef struct {
    int32_t tile, k_begin, k_end, role, peer_last;
} gemm_segment;

/* The work of logical workgroup wg in execution order; returns the number of
 * segments (may exceed max; only min(count, max) are written), or -1. */
int gemm_plan_segments(const gemm_plan *plan, int32_t wg, gemm_segment *out, int32_t max);

/* Output tile coordinates (tile row, tile column) of tile id t. */
int gemm_plan_tile_coords(const gemm_plan *plan, int32_t t, int32_t *tile_m, int32_t *tile_n);

/* Logical workgroup that hardware workgroup id hw runs (the XCD remap). */
int32_t gemm_plan_logical_wg(const gemm_plan *plan, int32_t hw);

/* Synchronously read the workspace status word written by the last run on
 * stream: 0 = ok, 1 = a fixup wait gave up (the output is not valid and the
 * workspace must be zero-filled again).  workspace NULL: the array that
 * gemm_run_noalloc uses on the current device.  Returns 0 or a negative
 * error. */
int gemm_workspace_status(const gemm_plan *plan, const void *workspace, void *stream,
                          int32_t *status);

/* One compiled kernel.  gemm_plan_create takes the first entry of the table
 * whose dtype, tile, bk, wave layout and stages match what the caller asked
 * for (0 = any) and whose copy hint matches GEMM_FLAG_STREAM_COPIES, so a plan
 * made with these fields runs exactly this kernel. */
typedef struct {
    int32_t dtype;          /* gemm_dtype */
    int32_t bm, bn, bk;
    int32_t wave_m, wave_n; /* wave grid of the workgroup */
    int32_t kind;           /* kernel_kind, as in gemm_plan_info */
    int32_t stages;
    int32_t stream_copies;  /* 1: needs GEMM_FLAG_STREAM_COPIES */
    int32_t threads;
    size_t lds_bytes;
} gemm_variant_info;

/* Number of compiled kernels. */
int32_t gemm_variant_count(void);

/* Kernel i (0 <= i < gemm_variant_count()) into *out; 0, or -1 on a bad
 * index or NULL out. */
int gemm_variant_get(int32_t i, gemm_variant_info *out);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_SK_H */
