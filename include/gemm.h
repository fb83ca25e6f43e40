/*
 * gemm.h - C ABI of the MI355X (gfx950) tiled dense matrix multiply.
 *
 *     D = A x B (+ C)
 *
 * Operation.  D is a separate M x N output and C an optional M x N addend
 * ("DCU K100 节点初探", section 5.2, MatMulAdd: D = sum + C; FlagGems "Hygon
 * optimization", section "DUMMA matrix instruction shapes": D = A x B + C).
 * A (M x K), B (K x N), C and D share one storage type, fp16 or bf16.
 * Products are accumulated in fp32 and the fp32 result (plus C, added once in
 * fp32 after the K loop) is rounded to the storage type, nearest-even
 * ("Hopper Support in Triton", slides 6-7: fp32 accumulator, fp16 x fp16 ->
 * fp32 dot, truncation to fp16 before the store).  No scale factors.
 *
 * Accuracy contract: every output d_ij is finite and
 *     |d_ij - ref_ij| <= ulp_out(ref_ij) + 2^-20 * sum_k |a_ik * b_kj|,
 * where ref_ij is the exact sum of the exact input values (plus c_ij) and
 * ulp_out is one unit in the last place of the storage type in the binade of
 * |ref_ij|.  For a fixed plan the result is bitwise reproducible run to run.
 *
 * Layout.  Every matrix is addressed by two element strides (row, column), as
 * in the pointer arithmetic of "Hopper Support in Triton", slide 6
 * (stride_am, stride_ak, stride_bk, stride_bn, stride_cm, stride_cn), through
 * which those slides reach any operand layout (slides 6 and 15, the block
 * pointers' strides).  Strides are >= 0 (GEMM_ERR_UNSUPPORTED otherwise).  C
 * and D must be row-major (column stride 1).  A and B may have any strides:
 *   - A row-major (stride_ak = 1) or stored K x M (stride_am = 1),
 *   - B row-major (stride_bn = 1) or stored N x K (stride_bk = 1),
 * run on the vector paths when the operand's contiguous extent and its other
 * stride are multiples of 8 elements and the bases are 16-byte aligned (the
 * four combinations give bitwise identical results for one tile
 * configuration); any other strides run on an element-wise path.
 *
 * Tiling.  The kernel walks a K loop over BLOCK_M x BLOCK_N x BLOCK_K tiles,
 * visits output tiles in GROUP_M bands for L2 reuse of B (FlagGems "Hygon
 * optimization", section "Grouped scheduling"), stages A/B tiles through an
 * LDS ring (section "Software pipelining"), and masks M/N/K tails with zero
 * fill ("Hopper Support in Triton", slides 15-16, k_remaining masks with
 * other = 0).  The tile configuration is chosen per (M, N, K, dtype, layout,
 * has_c) key ("Tuning Triton kernels", section 3: the key must name every dimension
 * the kernel tiles on), or forced by the caller.
 *
 * Ownership.  The caller owns A, B, C, D (device memory) and any plan.  The
 * library never allocates or frees device memory and never synchronizes:
 * gemm_run enqueues its kernels on the given stream and returns.  Errors in a
 * running kernel surface at the caller's next synchronization; launch
 * errors are returned as GEMM_ERR_HIP.  Plans are immutable after creation,
 * so one plan may be run concurrently on several streams.  Because gemm_run
 * only enqueues kernels (no allocation, memset or synchronization), a call
 * may be captured in a HIP graph and the graph replayed any number of times;
 * a K-sliced plan's workspace is prepared once, before the capture.
 *
 * Errors.  Every entry point returns a status and never aborts.  The detail of
 * the last failure on the calling thread is available from gemm_last_error().
 *
 * Streams are hipStream_t values passed as void* (NULL = the null stream).
 */
#ifndef DTG_GEMM_H
#define DTG_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM_ABI_VERSION 1

typedef enum gemm_dtype {
    GEMM_F16 = 0,   /* IEEE binary16 storage, fp32 accumulate */
    GEMM_BF16 = 1,  /* bfloat16 storage, fp32 accumulate */
    GEMM_I8 = 2     /* int8 A and B, int32 accumulate, int32 C and D (below) */
} gemm_dtype;

/* GEMM_I8 (FlagGems "Hygon optimization", section "DUMMA matrix instruction
 * shapes": the matrix unit takes integer inputs, which cover more k per
 * instruction): D[i][j] = sum_k A[i][k] B[k][j] (+ C[i][j]) modulo 2^32, as a
 * two's-complement int32 (the instruction's int32 accumulator wraps; the
 * exact sum is its residue whatever the order of addition).  A is int8 with
 * k contiguous (sa_k = 1: row-major M x K), B is int8 with k contiguous
 * (sb_k = 1: stored N x K, the layout of a weight matrix), C and D int32
 * row-major; strides in elements (bytes for A and B).  K, sa_m and sb_n must
 * be multiples of 16 and A, B 16-byte aligned; M and N are free.  Anything
 * else is GEMM_ERR_UNSUPPORTED (there is no element-wise int8 path), and so
 * are forced K slices.  The tile knobs keep their meaning with bk in pairs
 * of k (bk = 64 is a 128-deep K step) and mfma 16 / 32 selecting
 * v_mfma_i32_16x16x64_i8 / 32x32x32_i8. */

typedef enum gemm_status {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = 1,   /* bad size, pointer, stride, flag or overlap */
    GEMM_ERR_UNSUPPORTED = 2,   /* valid request this version does not run */
    GEMM_ERR_HIP = 3,           /* the HIP runtime reported an error */
    GEMM_ERR_WORKSPACE = 4      /* workspace missing or too small */
} gemm_status;

/* The problem.  Strides are in elements.  sc_* are ignored when has_c == 0. */
typedef struct gemm_problem {
    int64_t M, N, K;
    int64_t sa_m, sa_k;         /* A: element (i, k) at A[i*sa_m + k*sa_k] */
    int64_t sb_k, sb_n;         /* B: element (k, j) at B[k*sb_k + j*sb_n] */
    int64_t sc_m, sc_n;         /* C: element (i, j) at C[i*sc_m + j*sc_n] */
    int64_t sd_m, sd_n;         /* D: element (i, j) at D[i*sd_m + j*sd_n] */
    gemm_dtype dtype;
    int32_t has_c;              /* 1: D = A x B + C;  0: D = A x B */
} gemm_problem;

/* A tile configuration.  In a forced configuration a field of 0 means "the
 * planner's choice"; a plan reports every field filled in.
 *   bm, bn, bk    BLOCK_M, BLOCK_N, BLOCK_K
 *   stages        depth of the LDS ring (1 = single buffer)
 *   mfma          matrix instruction: 16 (16x16x32) or 32 (32x32x16)
 *   waves_m/_n    wavefront grid inside one workgroup (64 lanes per wave)
 *   group_m       GROUP_M of the grouped tile order (1 = row-major order)
 *   splitk        K slices across workgroups, summed in slice order by the
 *                 last workgroup to finish each output slab or tile (skinny
 *                 family; direct-to-LDS family for tiles of at most 64 fp32
 *                 accumulators per lane); needs a workspace when > 1; 1 for
 *                 the register-staged family.  Stream-K family: the number
 *                 of workgroups the (tile, K step) iterations are dealt to
 *                 (0 when forced: one per CU, each range >= 16 K steps)
 *   xcd_remap     GEMM_XCD_ON: pre-permute workgroup ids so each XCD gets a
 *                 contiguous band of the tile order; GEMM_XCD_OFF: plain ids
 *                 (0 in a forced configuration: the planner's choice)
 *   kernel        kernel family: 1 = register-staged tile kernel (any shape),
 *                 2 = skinny split-K kernel, 3 = direct-to-LDS tile kernel
 *                 (when M fits one row of its 64 x 64 tiles, the variant that
 *                 loads B non-temporal: gemm_plan_describe names it),
 *                 6 = direct-to-LDS stream-K kernel (row-major A and B; the
 *                 K steps of all tiles dealt out evenly to `splitk`
 *                 workgroups, tiles cut between workgroups summed from fp32
 *                 parts in a workspace, in part order, by the last to finish;
 *                 "Hopper Support in Triton", the SplitK / stream-K slides) */
#define GEMM_XCD_ON 1
#define GEMM_XCD_OFF 2

typedef struct gemm_config {
    int32_t bm, bn, bk;
    int32_t stages;
    int32_t mfma;
    int32_t waves_m, waves_n;
    int32_t group_m;
    int32_t splitk;
    int32_t xcd_remap;
    int32_t kernel;
} gemm_config;

/* Device facts the planner uses.  gemm_device_query fills it from the HIP
 * runtime; tests may pass a hand-made one to gemm_plan_create_for. */
typedef struct gemm_device_info {
    int32_t arch;               /* gfx number, 950 for MI355X */
    int32_t cu_count;           /* compute units */
    int32_t xcd_count;          /* accelerator dies sharing the grid */
    int32_t clock_khz;          /* peak engine clock */
    int64_t lds_per_cu;         /* LDS bytes per CU */
    int64_t lds_per_wg;         /* max LDS bytes one workgroup may allocate */
    int32_t wave_size;          /* lanes per wavefront */
} gemm_device_info;

typedef struct gemm_plan gemm_plan;   /* opaque, immutable after creation */

/* Fill *info for HIP device `device`.  GEMM_ERR_HIP without a usable device. */
gemm_status gemm_device_query(int device, gemm_device_info* info);

/* Validate *prob and choose a configuration for HIP device `device` (queried
 * once per device and cached).  force may be NULL; its non-zero fields
 * override the planner.  A forced configuration the kernels cannot run (LDS
 * over the device limit, tile not a multiple of the instruction and wave
 * grid, unsupported combination) is GEMM_ERR_UNSUPPORTED.  No device work. */
gemm_status gemm_plan_create(const gemm_problem* prob, int device,
                             const gemm_config* force, gemm_plan** out);

/* Same as gemm_plan_create with explicit device facts; touches no device.
 * A plan made this way runs only on a device with the same facts. */
gemm_status gemm_plan_create_for(const gemm_problem* prob, const gemm_device_info* info,
                                 const gemm_config* force, gemm_plan** out);

/* Free a plan.  NULL is a no-op. */
void gemm_plan_destroy(gemm_plan* plan);

/* The configuration a plan will run. */
gemm_status gemm_plan_config(const gemm_plan* plan, gemm_config* out);

/* Launch geometry of a plan: grid (workgroups), threads per workgroup and
 * LDS bytes per workgroup. */
gemm_status gemm_plan_launch(const gemm_plan* plan, int64_t* grid, int32_t* threads,
                             int64_t* lds_bytes);

/* A one-line, NUL-terminated description of the plan (configuration, grid,
 * LDS, kernel name) written into buf[0..len).  Truncates to fit. */
gemm_status gemm_plan_describe(const gemm_plan* plan, char* buf, size_t len);

/* Device workspace the plan needs in bytes (0 unless the plan splits K across
 * workgroups).  Layout: a fixed 16 KiB region of per-slab arrival counters,
 * then the fp32 partial tiles. */
gemm_status gemm_workspace_size(const gemm_plan* plan, size_t* bytes);

/* Prepare a workspace for a plan: enqueue on `stream` a kernel that zero-fills
 * it.  Required once before the first gemm_run with that workspace (a
 * zero-filled allocation needs nothing more); every launch leaves its counters
 * zero again, so the workspace can be reused for any number of runs of plans
 * whose workspace size fits (the counters sit in a fixed region shared by all
 * plans).  One workspace serves one launch at a time: runs
 * that overlap in time (other streams) need separate workspaces.
 * GEMM_ERR_WORKSPACE if it is NULL or smaller than gemm_workspace_size. */
gemm_status gemm_workspace_init(const gemm_plan* plan, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Enqueue D = A x B (+ C) on `stream`.  A, B, D are device pointers; C is a
 * device pointer when the plan's problem has has_c = 1 and must be NULL
 * otherwise.  D may equal C when their strides are equal (in place D += AxB);
 * any other overlap of D with A, B or C is GEMM_ERR_INVALID_ARG.  workspace
 * may be NULL when gemm_workspace_size reports 0; otherwise it must be at
 * least that many bytes, 256-byte aligned and prepared by gemm_workspace_init
 * (else GEMM_ERR_WORKSPACE).  M = 0 or N = 0 launches nothing; K = 0 writes
 * D = C (or zeros). */
gemm_status gemm_run(const gemm_plan* plan, const void* A, const void* B, const void* C,
                     void* D, void* workspace, size_t workspace_bytes, void* stream);

/* Largest workspace, in bytes, that gemm_run_static provides (24 MiB). */
#define GEMM_STATIC_SCRATCH_BYTES (24u * 1024u * 1024u)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): gemm_run
 * with the plan's workspace taken from a fixed device array of
 * GEMM_STATIC_SCRATCH_BYTES that each device the library runs on holds until
 * the process ends.  Allocates nothing and calls no allocating routine.  A, B,
 * C, D and stream as for gemm_run; the kernels run on the stream's device.
 * A plan whose gemm_workspace_size is 0 runs exactly as gemm_run.  The first
 * call on a device looks the array up (with that device current) and
 * zero-fills its counter region on `stream`; every launch leaves the counters
 * at zero again.  GEMM_ERR_WORKSPACE (before any device call) if the plan's
 * workspace exceeds GEMM_STATIC_SCRATCH_BYTES.  All calls on one device share
 * the array: calls that overlap in time on one device (several streams or
 * threads) race, and the caller must serialize them. */
gemm_status gemm_run_static(const gemm_plan* plan, const void* A, const void* B, const void* C,
                            void* D, void* stream);

/* One call: plan (cached per problem key and device, thread-safe) and run on
 * the current HIP device.  strides = {sa_m, sa_k, sb_k, sb_n, sc_m, sc_n,
 * sd_m, sd_n}.  Plans needing a workspace are not chosen here. */
gemm_status gemm(const void* A, const void* B, const void* C, void* D,
                 int64_t M, int64_t N, int64_t K, const int64_t strides[8],
                 gemm_dtype dtype, int32_t has_c, void* stream);

/* Release every plan cached by gemm().  Not safe concurrently with gemm(). */
void gemm_cache_clear(void);

/* Bytes of one A/B tile pair staged per pipeline stage, summed over stages:
 * stages * (bm + bn) * bk * element bytes, bk in elements of dtype (2 bytes,
 * or 1 for GEMM_I8) (FlagGems "Hygon optimization",
 * section "Software pipelining": (BLOCK_M + BLOCK_N) x BLOCK_K x 2 bytes per
 * pair, 8 KiB at 64 x 64 x 32 fp16).  Returns -1 on a bad argument. */
int64_t gemm_lds_bytes(int32_t bm, int32_t bn, int32_t bk, int32_t stages, gemm_dtype dtype);

/* The output tile (pid_m, pid_n) that workgroup `wg` of a launch over
 * num_pid_m x num_pid_n tiles computes, after the optional XCD pre-permutation
 * (xcd_count > 1) and the GROUP_M band order.  The kernels use the same code.
 * Returns GEMM_ERR_INVALID_ARG for wg outside the grid. */
gemm_status gemm_tile_of_workgroup(int64_t wg, int64_t num_pid_m, int64_t num_pid_n,
                                   int32_t group_m, int32_t xcd_count,
                                   int64_t* pid_m, int64_t* pid_n);

/* The stream-K schedule of a kernel-6 plan, as the kernel computes it: the
 * pieces of workgroup range `wg` (after the XCD pre-permutation) when
 * tiles x k_steps iterations are dealt to `workgroups` ranges, range w being
 * [floor(w T / W), floor((w + 1) T / W)) of T = tiles x k_steps.  Piece p
 * fills out[6p .. 6p + 5] with: tile (grouped order), first and end K step,
 * part number, the tile's part count (1: whole tile, written directly),
 * and the workspace slot of that part (-1 for a whole tile).  At most
 * max_pieces are written; *count gets the range's piece count.
 * GEMM_ERR_INVALID_ARG unless 0 <= wg < workgroups <= tiles x k_steps and
 * tiles x k_steps x workgroups < 2^31. */
gemm_status gemm_streamk_pieces(int32_t tiles, int32_t k_steps, int32_t workgroups, int32_t wg,
                                int32_t* out, int32_t max_pieces, int32_t* count);

const char* gemm_status_string(gemm_status status);

/* Detail of the last failure on this thread ("" if none). */
const char* gemm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DTG_GEMM_H */
