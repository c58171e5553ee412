/*
 * mswz_gemm.h — C ABI of the swizzled-operand GEMM library for AMD Instinct
 * MI355X (gfx950), libmswz.so.
 *
 * The operation (tcgen05.mma page, "Operands and repeat axes", "Shared
 * descriptors are byte-stride contracts" and "Example: four K16 issues for a
 * 128x64x64 product"):
 *
 *     D[m][n] = beta * D[m][n] + sum_k a(m,k) * b(n,k)          (dense)
 *
 * i.e. D = A . B^T with B held as (N,K), fp32 accumulation, fp32 (or rounded
 * bf16 / fp16) output.  `beta`
 * is the page's `accum` flag: 0 overwrites D (its old contents are never read,
 * so NaNs in it do not propagate), 1 accumulates onto it.  Block-scaled
 * operands (same page, "Weight-stationary and block scaling") attach one
 * scale byte per row and per `scale_vec_len` consecutive K elements:
 *
 *     D[m][n] = beta * D[m][n]
 *             + sum_k (2^(SFA[m][k/V]-127) a(m,k)) * (2^(SFB[n][k/V]-127) b(n,k))
 *
 * Storage (all tensors contiguous, row-major, device memory):
 *     A  K-major: [M][K]      A  MN-major: [K][M]     ("K-major rows enumerate
 *     B  K-major: [N][K]      B  MN-major: [K][N]      M/N, MN-major rows K")
 *     (E2M1: K-major only, [M][K/2] and [N][K/2] bytes, two elements a byte;
 *      E2M3 / E3M2: K-major only, [M][K] and [N][K] bytes, each 16-byte block
 *      holding sixteen 6-bit values, value j in bits 6j .. 6j+5 of the block's
 *      first twelve bytes taken little-endian, the last four bytes padding
 *      that is never read: the padded FP6 form of the tcgen05.cp page's
 *      "Native FP4/FP6 decompression"; E2M1_P64: the padded FP4 form of the
 *      same section, [M][K] and [N][K] bytes, each 16-byte block holding
 *      sixteen 4-bit values in its first eight bytes, value j in the low
 *      (j even) or high (j odd) nibble of byte j/2, then eight padding bytes)
 *     D  [M][N] in the plan's d_dt (fp32, bf16 or fp16)
 *     SFA uint8 [M][K/V], SFB uint8 [N][K/V]: OCP E8M0 exponents, value 2^(E-127)
 *       (or [K/V][M] and [K/V][N] after gemm_plan_set_scale_major)
 * Element formats: fp16 (IEEE binary16), bf16, fp8 = OCP E4M3 (bias 7, no
 * infinities), fp4 = OCP E2M1 (bias 1, no infinities or NaN; the pages'
 * "four-bit values"), fp6 = OCP E2M3 (bias 1) or E3M2 (bias 3), neither with
 * infinities or NaN (the pages' "six-bit values").  Results are fp32 sums of exact products; the summation order
 * is fixed per plan, so a plan gives bit-identical results run to run.
 *
 * Ownership: the caller owns every device buffer and the stream.  A plan holds
 * host metadata only and is immutable once created (apart from its scale
 * layout, gemm_plan_set_scale_major), so one plan may be used from several
 * host threads and streams at once.  gemm_run* enqueue their
 * kernels on `stream` (one; two for gemm_run_ws's split path) and return; they
 * allocate nothing, do not synchronise and keep no pointer.  Buffers must stay alive until the stream has passed the kernel
 * (the pages' rule of keeping allocations alive until consumers complete).
 * Scales are prepared by the caller in the layout above; supplying them does
 * not change the plan.
 *
 * Errors: every call returns an int status (MSWZ_OK or a negative code);
 * nothing is printed and there is no fallback path.  Layout requirements are
 * checked against the explicit arguments and nothing is inferred: shapes the
 * plan cannot tile, unsupported dtype or major combinations, misaligned or
 * null pointers and beta outside {0,1} are rejected before any GPU work.
 */
#ifndef MSWZ_GEMM_H
#define MSWZ_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MSWZ_OK = 0,
    MSWZ_ERR_INVALID = -1,      /* bad argument: size <= 0, null pointer, beta not 0/1, bad enum */
    MSWZ_ERR_UNSUPPORTED = -2,  /* valid request this library has no kernel for (shape not a tile multiple, dtype/major combination) */
    MSWZ_ERR_ALIGN = -3,        /* pointer not 16-byte aligned */
    MSWZ_ERR_HIP = -4,          /* the HIP runtime reported an error on launch */
    MSWZ_ERR_KIND = -5,         /* dense plan passed to gemm_run_blockscaled or the reverse */
    MSWZ_ERR_SCRATCH = -6       /* gemm_run_ws_noalloc: the plan needs more than the library's scratch */
} mswz_status;

typedef enum {
    MSWZ_DT_F16 = 1,
    MSWZ_DT_BF16 = 2,
    MSWZ_DT_E4M3 = 3,
    MSWZ_DT_F32 = 4,
    MSWZ_DT_E2M1 = 5,           /* OCP FP4, two per byte, element 2j in the low nibble of byte j */
    MSWZ_DT_E2M3 = 6,           /* OCP FP6 E2M3, sixteen per 16-byte block (see Storage) */
    MSWZ_DT_E3M2 = 7,           /* OCP FP6 E3M2, sixteen per 16-byte block (see Storage) */
    MSWZ_DT_E2M1_P64 = 8        /* OCP FP4 E2M1, sixteen per 16-byte block (see Storage) */
} mswz_dtype;

typedef enum {
    MSWZ_MAJOR_K = 0,
    MSWZ_MAJOR_MN = 1
} mswz_major;

typedef struct gemm_plan gemm_plan;

/*
 * Create a plan for one problem shape.
 *   out           receives the plan (set to NULL on failure)
 *   M, N, K       problem sizes, each > 0
 *   a_dt, b_dt    operand element formats
 *   d_dt          MSWZ_DT_F32, or MSWZ_DT_BF16 / MSWZ_DT_F16: the fp32 result
 *                 rounded to nearest even into D's format (beta = 1 then
 *                 reads D in that format and adds it in fp32 before
 *                 rounding); narrow D always uses the 256 tile
 *                 Supported: (F16,F16), (BF16,BF16) dense; (E4M3,E4M3) and
 *                 (E2M1,E2M1), (E2M3,E2M3), (E3M2,E3M2), (E2M1_P64,E2M1_P64)
 *                 block-scaled, any mix of E4M3, E2M3, E3M2 and E2M1_P64
 *                 for A and B, and (E4M3,E2M1), (E2M1,E4M3) (the pages' mixed
 *                 f8f6f4 kind; each operand decoded in its own format, 256
 *                 tile).
 *   a_major       MSWZ_MAJOR_K or MSWZ_MAJOR_MN (MN only for 16-bit formats)
 *   b_major       MSWZ_MAJOR_K or MSWZ_MAJOR_MN (MN only for 16-bit formats)
 *   scale_vec_len 0 for dense; 32 (one scale per 32 K elements) for E4M3, E2M1,
 *                 E2M3, E3M2 and E2M1_P64; or 16 (one scale per 16 K
 *                 elements: the pages' scale_vec::4X) for E2M1, E2M1_P64,
 *                 E2M3 and E3M2 with A and B of the same kind
 * Shape rules: block-scaled K: any multiple of scale_vec_len (E2M1: of 32 as
 * well, so that rows of K/2 bytes stay 16-byte aligned; E4M3 with dense E2M1:
 * a multiple of 256, as that kernel stages the E2M1 operand two of the E4M3
 * operand's 128-element steps at a time); a K that is not a
 * multiple of the kernel's K step (128 elements; E2M1 256) uses the 256 tile,
 * whose last K step reads the values beyond K as zeros and gives their scale
 * blocks the exponent 127 (the scale array itself holds K/V bytes per row,
 * nothing beyond them is read).  E2M1, E2M3, E3M2, E2M1_P64 and mixed kinds
 * always use the 256 tile.  16-bit K: any K with K % 8 == 0 (16-byte K-major rows; any
 * K when both operands are MN-major); a K that is not a multiple of 64 uses
 * the 256 tile, whose last K step reads the values beyond K as zeros.  M and N
 * multiples of 64 choose among 256, 128 and 64 square tiles; otherwise (tails)
 * the 256 tile is used with masked stores, and N % 4 == 0 is required (16-byte
 * rows of D), as well as M % 8 == 0 for MN-major A and N % 8 == 0 for MN-major
 * B.  MN-major operands must be smaller than 4 GiB - 256 bytes.  A 16-bit
 * K-major A with M <= 64, N % 64 == 0 and K % 1024 == 0 (K-major B, fp32 D,
 * packed storage) selects the weight-streaming kernel (M padded to 32 or 64
 * rows, the padding never read from memory nor stored).
 * Returns MSWZ_OK, MSWZ_ERR_INVALID or MSWZ_ERR_UNSUPPORTED.
 */
int gemm_plan_create(gemm_plan **out, int64_t M, int64_t N, int64_t K,
                     int a_dt, int b_dt, int d_dt, int a_major, int b_major,
                     int32_t scale_vec_len);

/*
 * gemm_plan_create for operands and D stored with a row pitch, so that each
 * can be a view into a wider matrix (tcgen05.mma page, "Shared descriptors are
 * byte-stride contracts": the layout is given by explicit strides, 16-byte
 * multiples, and checked, never inferred).
 *   lda   elements from one stored row of A to the next: a K-major A is
 *         [M][lda] with lda >= K, an MN-major A is [K][lda] with lda >= M
 *   ldb   the same for B ([N][ldb], ldb >= K; or [K][ldb], ldb >= N)
 *   ldd   elements from one row of D to the next, ldd >= N
 * 0 for any of them means packed (K, M / N, N).  A plan with any pitch other
 * than packed uses the 256 tile and needs every stored row 16-byte aligned:
 * lda and ldb multiples of 8 (16-bit), 16 (E4M3, E2M3, E3M2, E2M1_P64: whole
 * 16-byte blocks) or 32 (E2M1), ldd a multiple
 * of 4; pitches are at most 2^22, and an MN-major operand's span
 * ((K - 1) * ld + M or N elements) must stay below 4 GiB.  The elements
 * between a row's end and the next row's start are neither read (operands)
 * nor written (D).  Scale arrays stay packed.  Other arguments and the
 * returns are those of gemm_plan_create, which is this function with three
 * zero pitches.
 */
int gemm_plan_create_ld(gemm_plan **out, int64_t M, int64_t N, int64_t K,
                        int a_dt, int b_dt, int d_dt, int a_major, int b_major,
                        int32_t scale_vec_len, int64_t lda, int64_t ldb,
                        int64_t ldd);

/*
 * Scale layout of a block-scaled plan.  The tcgen05.mma page ("Operands and
 * repeat axes", the SFA / SFB rows of its shape table) gives the scale
 * operands the K-repeat axis outside their rows; this call lets SFA and SFB
 * be stored in that order.
 *   sf_major  MSWZ_MAJOR_K (the plan's default): SFA uint8 [M][K/V], SFB
 *             [N][K/V], each row's scales consecutive.  MSWZ_MAJOR_MN: SFA
 *             uint8 [K/V][M], SFB [K/V][N], each K block's scales of all rows
 *             consecutive (M, resp. N, bytes per K block).  Values and the
 *             product are the same; only the addresses differ.
 * MN-major scales are taken with V = 32, K a multiple of the K step (128;
 * 256 for dense E2M1), M and N multiples of 16, K/V * M and K/V * N at most
 * 2^31 (bytes of each scale array), any D, and A and B each one of E4M3,
 * E2M3, E3M2 and padded E2M1 (mixed or not), dense E2M1 on both sides, or
 * E4M3 A with dense E2M1 B (K a multiple of 256); not dense E2M1 A with
 * E4M3 B, not 16-element blocks.  Such a plan runs the 256x256 tile (gemm_plan_describe shows
 * it); setting MSWZ_MAJOR_K again restores the variant chosen at creation.
 * The plan is changed in place: not while a call on it is being enqueued.
 * Returns MSWZ_OK, MSWZ_ERR_INVALID (NULL plan, unknown sf_major),
 * MSWZ_ERR_KIND (a dense plan) or MSWZ_ERR_UNSUPPORTED (MN-major for any
 * other configuration; the plan is left unchanged).
 */
int gemm_plan_set_scale_major(gemm_plan *plan, int sf_major);

/*
 * Enqueue D = beta*D + A.B^T for a dense plan on `stream` (a hipStream_t;
 * NULL is the default stream): the product of the tcgen05.mma page's
 * "Operands and repeat axes" and "Example: four K16 issues for a 128x64x64
 * product" (B held as (N,K), fp32 accumulation, `accum` as beta), with the
 * operand majors of its "Shared descriptors are byte-stride contracts".
 * A, B, D are device pointers, 16-byte aligned, in the layouts above; the
 * caller owns them and keeps them alive until the stream passes the kernel.
 * Returns MSWZ_OK, MSWZ_ERR_INVALID (null pointer, beta not 0 or 1),
 * MSWZ_ERR_ALIGN, MSWZ_ERR_KIND (a block-scaled plan) or MSWZ_ERR_HIP (launch
 * error); on any error other than MSWZ_ERR_HIP nothing was enqueued.
 */
int gemm_run(const gemm_plan *plan, const void *A, const void *B, void *D,
             int beta, void *stream);

/*
 * Device workspace, in bytes, that gemm_run_ws can use for this plan: > 0 for
 * weight-streaming plans (the skinny kernel above) with N % 256 == 0 (K split
 * into S parts, each a multiple of 256: the smallest power of two up to 16
 * giving N/256 * S >= 256 workgroups, else the largest that fits): S * M * N * 4
 * bytes of fp32 partials; 0 otherwise.
 * MSWZ_ERR_INVALID for a NULL plan.
 */
int64_t gemm_plan_workspace_size(const gemm_plan *plan);

/*
 * gemm_run with a caller-provided device workspace (tcgen05.mma page,
 * "Weight-stationary and block scaling": the weight-stationary workload,
 * read here as a few rows of activations against a large weight matrix that
 * is streamed once).  For a plan with gemm_plan_workspace_size(plan) > 0 it
 * splits K over S workgroups per 256 output columns, each storing an fp32
 * partial in the workspace, and enqueues a second kernel that sums the S
 * partials of every output in a fixed order and applies beta; results are
 * bit-identical run to run (not necessarily to gemm_run's, whose summation
 * order differs).  For other plans it is gemm_run and ignores the workspace.
 *   workspace        device pointer, 16-byte aligned, at least
 *                    gemm_plan_workspace_size(plan) bytes; the caller owns it.
 *                    Its contents before the call do not matter (every byte
 *                    the reduction reads is written first by the same call).
 *                    Two calls that may run at the same time must not share
 *                    a workspace.
 *   workspace_bytes  its size.
 * Returns as gemm_run; MSWZ_ERR_INVALID also for a NULL or too small workspace.
 */
int gemm_run_ws(const gemm_plan *plan, const void *A, const void *B, void *D,
                int beta, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * gemm_run_ws for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results as gemm_run_ws, bit for bit, with the fp32
 * partials in a scratch array the library owns, gemm_noalloc_scratch_bytes()
 * bytes (16 MiB, enough for the 64 x 16384 x 8192 weight-streaming shape) per
 * GPU, held until the process ends.  It calls no hipMalloc, hipFree or other
 * allocating routine; the first call on a device looks the array's device
 * address up (hipGetSymbolAddress) with that device current, so `stream` must
 * belong to the current device.  Every call on one GPU shares that GPU's
 * array: calls that may overlap on one GPU (other streams, other host
 * threads) race and must not be issued.  Plans without a split path run as
 * gemm_run and use no scratch.
 * Returns as gemm_run_ws, and MSWZ_ERR_SCRATCH (before any GPU work) when
 * gemm_plan_workspace_size(plan) exceeds the scratch size.
 */
int gemm_run_ws_noalloc(const gemm_plan *plan, const void *A, const void *B, void *D,
                        int beta, void *stream);

/* Bytes of the scratch array gemm_run_ws_noalloc uses per GPU. */
int64_t gemm_noalloc_scratch_bytes(void);

/*
 * Enqueue the block-scaled product for a plan created with scale_vec_len > 0
 * (tcgen05.mma page, "Weight-stationary and block scaling": one scale vector
 * per row of A and of B, each scale covering scale_vec_len consecutive K
 * elements; every element is multiplied by 2^(E-127) of its block before the
 * products are summed).  SFA [M][K/V] and SFB [N][K/V] are device pointers to
 * E8M0 bytes, 16-byte aligned, owned by the caller.  Same returns as
 * gemm_run, with MSWZ_ERR_KIND for a dense plan.
 */
int gemm_run_blockscaled(const gemm_plan *plan, const void *A, const void *B,
                         const uint8_t *SFA, const uint8_t *SFB, void *D,
                         int beta, void *stream);

/*
 * Per-call options (tcgen05.mma page, "Weight-stationary and block scaling":
 * neg_a, neg_b, sat_d, the dense disable-output-lane masks, the zero-column
 * mask of the weight-stationary form, and pred are explicit parameters; the
 * page names them without defining them, so the readings are stated here).
 */
typedef struct {
    int neg_a, neg_b;           /* nonzero: A (B) enters negated; the product's sign
                                   is (-1)^(neg_a + neg_b) (negation is exact) */
    int sat_d;                  /* nonzero: every stored D value is clamped to D's
                                   largest finite magnitude (fp32 3.40282347e38,
                                   bf16 3.38953139e38, fp16 65504), infinities
                                   included; NaN is stored unchanged */
    const uint32_t *row_mask;   /* device pointer or NULL: ceil(M/32) words; bit m % 32
                                   of word m / 32 set leaves row m of D untouched
                                   (not written; its old value does not enter any result) */
    const uint32_t *col_zero;   /* device pointer or NULL: ceil(N/32) words; bit n % 32
                                   of word n / 32 set makes column n of the product
                                   zero (row n of B treated as zero), so that column
                                   of D becomes beta * D */
    int pred;                   /* zero: nothing is enqueued and D is unchanged (the
                                   arguments are still checked first) */
} gemm_opts;

/*
 * gemm_run / gemm_run_blockscaled with options.  SFA and SFB must be NULL for
 * a dense plan and non-NULL for a block-scaled one.  opts == NULL, or options
 * that change nothing (neg_a == neg_b, no saturation, no masks, pred != 0),
 * run exactly as gemm_run / gemm_run_blockscaled.  Otherwise the call runs
 * on the 256x256 tile whatever tile the plan chose (any plan's shape is
 * valid for it); the masks are read once per output row / column group and
 * must be 4-byte aligned (else MSWZ_ERR_ALIGN).  Returns as gemm_run, and
 * MSWZ_ERR_INVALID for scale pointers that do not match the plan.  Calls with
 * options that change something are asynchronous like gemm_run and allocate
 * nothing; the masks must stay alive until the stream passes the kernel.
 */
int gemm_run_opts(const gemm_plan *plan, const void *A, const void *B,
                  const uint8_t *SFA, const uint8_t *SFB, void *D, int beta,
                  const gemm_opts *opts, void *stream);

/* Release a plan (NULL is allowed). */
void gemm_plan_destroy(gemm_plan *plan);

/* Static description of a status code (never NULL). */
const char *gemm_status_str(int status);

/*
 * Launch geometry a plan chose, for reporting: fills up to `n` of
 * {variant, tile_m, tile_n, tile_k, threads_per_block, blocks, lds_bytes,
 *  group_m} and returns how many it wrote, or a negative status.
 */
int gemm_plan_describe(const gemm_plan *plan, int64_t *info, int n);

/*
 * Address functions the kernels use, exported for host-side checking (no GPU
 * work).  mswz_desc_address is the pages' shared-descriptor walk (tcgen05.cp
 * page, "Shared descriptor address walk"; tcgen05.mma page, "Shared
 * descriptors are byte-stride contracts"): the physical byte address of
 * 32-bit word w of row r for (ldo, sdo, swizzle mode 0..4, major, origin).
 * mswz_desc_check returns 0 when (ldo, sdo, mode, origin) satisfy the pages'
 * descriptor rules, else the number of the first rule broken.
 * mswz_tile_offset is the byte offset of 16-byte chunk `chunk` (0..7) of row
 * `row` in the kernels' LDS operand tile (128-byte rows).
 */
/*
 * The kernels' workgroup -> output tile map (XCD-aware raster): tile
 * (tile_m, tile_n) of a tiles_m x tiles_n grid computed by workgroup `block`
 * for the raster parameter group_m (the value gemm_plan_describe reports).
 * Returns MSWZ_OK, or MSWZ_ERR_INVALID for arguments outside the grid.
 */
int mswz_tile_of_block(int block, int tiles_m, int tiles_n, int group_m,
                       int *tile_m, int *tile_n);

/*
 * The 256x256 kernel's per-lane LDS addresses for one wave-wide access, from
 * the same address functions the kernel uses (no GPU work), so that host
 * tests can check the staging layouts and fragment maps bit for bit.
 * Offsets are bytes from the start of the operand tile (or of the scale
 * stage, or of a wave's epilogue area).  Writes `count` values to out (at
 * most n) and returns count, or MSWZ_ERR_INVALID.
 *   MSWZ_LDS_DMA_K      p0 = copy instruction q (0..31): out[2l] = LDS offset
 *                       lane l writes (16 bytes), out[2l+1] = the source
 *                       offset row * 128 + 16 * chunk in the step's [256][128 B]
 *                       slice of the operand                   (count 128)
 *   MSWZ_LDS_DMA_MN     p0 = q (0..31): the same for an MN-major operand, source
 *                       k * 512 + 16 * chunk in the step's [64][512 B] slice
 *   MSWZ_LDS_FRAG_K16   p0 = 16-row block b (0..15), p1 = sub-step (0..1): the
 *                       16-byte read of a 16-bit K-major 16x16x32 fragment (64)
 *   MSWZ_LDS_FRAG_MN16  p0 = b, p1 = sub-step: the two 8-byte transposing
 *                       reads (ds_read_b64_tr_b16) of an MN-major fragment (128)
 *   MSWZ_LDS_FRAG_E4M3  p0 = b (0..15): the two 16-byte reads (bytes 0..15 and
 *                       16..31) of an E4M3 fragment                     (128)
 *   MSWZ_LDS_FRAG_PAD   p0 = b: the two 16-byte reads of a padded 6- or
 *                       4-bit fragment                                   (128)
 *   MSWZ_LDS_FRAG_E4M3_MIXED  p0 = b: E4M3 paired with a padded kind     (128)
 *   MSWZ_LDS_FRAG_E2M1  p0 = b, p1 = sub-step (0..1): the 16-byte read of a
 *                       dense E2M1 fragment (paired with E4M3: p1 = the
 *                       half of its two-step tile row)                    (64)
 *   MSWZ_LDS_FRAG_E4M3_FP4  p0 = b: the two 16-byte reads of an E4M3
 *                       fragment paired with dense E2M1                  (128)
 *   MSWZ_LDS_SCALE_GRP  p0 = b (0..7), p1 = step in its group of four (0..3):
 *                       the scale byte each lane reads (A side, wave rows 0..127)
 *   MSWZ_LDS_SCALE_DMA  p0 = wave (0..7): out[2l] = stage offset lane l writes
 *                       (16 bytes), out[2l+1] = the row of its 64-row group
 *                       whose four steps' scale bytes it copies        (128)
 *   MSWZ_LDS_SCALE_GRP_WIDE  p0 = b (0..7), p1 = step in its group of eight
 *                       (0..7): the scale byte each lane reads from the
 *                       32-byte-per-row stage (6-bit kinds; A side)       (64)
 *   MSWZ_LDS_SCALE_DMA_WIDE  p0 = wave (0..7), p1 = copy (0..1): out[2l] =
 *                       stage offset lane l writes (16 bytes), out[2l+1] =
 *                       2 x (row of the wave's 64-row group) + the half of
 *                       its 32 scale bytes it copies (slot order of the 6-bit
 *                       kinds)                                          (128)
 *   MSWZ_LDS_SCALE_DMA_WIDE_NAT  the same for dense E2M1 (rows in order)  (128)
 *   MSWZ_LDS_SCALE_FP4_WIDE  p0 = b (0..7), p1 = 2 x step in its group of
 *                       four + sub-step (0..7): the scale byte each lane
 *                       reads (dense E2M1, A side)                        (64)
 *   MSWZ_LDS_SCALE_DMA_MN  p0 = wave (0..7), p1 = copy (0..1), MN-major
 *                       scales: out[2l] = stage offset lane l writes (16
 *                       bytes; B's half from 8192), out[2l+1] = 256 x (K block
 *                       of the 32-block group) + first of the 16 rows whose
 *                       scales for that block it copies                  (128)
 *   MSWZ_LDS_SCALE_GRP_MN  p0 = b (0..7), p1 = step in its group of eight
 *                       (0..7): the scale byte each lane reads, MN-major
 *                       scales (E4M3 and padded kinds; A side, wave rows
 *                       0..127)                                           (64)
 *   MSWZ_LDS_SCALE_FP4_MN  p0 = b (0..7), p1 = 2 x step in its group of
 *                       four + sub-step (0..7): the same for dense E2M1   (64)
 *   MSWZ_LDS_EPI_WRITE  p0 = quarter q (0..3), p1 = 16*rows + 4*ii + j: the
 *                       16-byte write of 16x16 block (2q + ii, j); rows 0:
 *                       16-bit, 1: split-row fragments on both sides (E4M3,
 *                       padded kinds), 2: on the M side only (E4M3 A with
 *                       dense E2M1 B), 3: on the N side only            (64)
 *   MSWZ_LDS_EPI_READ   p0 = read-back instruction k (0..7)              (64)
 */
enum {
    MSWZ_LDS_DMA_K = 1, MSWZ_LDS_DMA_MN = 2, MSWZ_LDS_FRAG_K16 = 3, MSWZ_LDS_FRAG_MN16 = 4,
    MSWZ_LDS_FRAG_E4M3 = 5, MSWZ_LDS_FRAG_PAD = 6, MSWZ_LDS_FRAG_E4M3_MIXED = 7, MSWZ_LDS_FRAG_E2M1 = 8,
    MSWZ_LDS_SCALE_GRP = 9, MSWZ_LDS_SCALE_DMA = 10, MSWZ_LDS_EPI_WRITE = 11, MSWZ_LDS_EPI_READ = 12,
    MSWZ_LDS_FRAG_E4M3_FP4 = 13, MSWZ_LDS_SCALE_GRP_WIDE = 14, MSWZ_LDS_SCALE_DMA_WIDE = 15,
    MSWZ_LDS_SCALE_DMA_WIDE_NAT = 16, MSWZ_LDS_SCALE_FP4_WIDE = 17, MSWZ_LDS_SCALE_DMA_MN = 18,
    MSWZ_LDS_SCALE_GRP_MN = 19, MSWZ_LDS_SCALE_FP4_MN = 20
};
int mswz_lds_lanes(int pattern, int p0, int p1, uint32_t *out, int n);

int64_t mswz_desc_address(int64_t r, int64_t w, int64_t ldo, int64_t sdo,
                          int mode, int major, int64_t origin);
int mswz_desc_check(int64_t ldo, int64_t sdo, int mode, int64_t origin);
uint32_t mswz_tile_offset(uint32_t row, uint32_t chunk);

#ifdef __cplusplus
}
#endif

#endif /* MSWZ_GEMM_H */
