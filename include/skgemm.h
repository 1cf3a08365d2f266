/*
 * skgemm.h -- C ABI of the stream-K GEMM / conv-wgrad engine for gfx950.
 *
 * One library, libskgemm.so, serves two workloads with one tiled MFMA
 * engine:
 *   - GEMM in the "rcr" layout (row-major A, column-major B, row-major C) on
 *     fp16, bf16 or OCP fp8 e4m3 inputs with optional per-row A and
 *     per-column B fp32 scales, fp32 accumulation;
 *   - backward-weight convolution (wgrad) of NHWC activations as an implicit
 *     GEMM whose M is the output channels (conv groups folded into M per
 *     group), N the filter taps times input channels of a group, and whose
 *     reduction runs over every output pixel of every image.
 *
 * Output tiles are split by a host planner into a data-parallel set (whole
 * waves of the CTA pool) and a stream-K remainder whose MAC iterations are
 * spread as contiguous, balanced ranges over the pool (rocm-libraries PR
 * #13151 "feat(rocke): stream-K for implicit-GEMM conv wgrad", Technical
 * Details: Partitioner).  Tiles shared by several CTAs are fixed up in one of
 * four ways (same PR, Technical Details: Wgrad kernel): linear and tree are
 * deterministic hand-offs through per-(CTA, wave) flags with device-scope
 * release/acquire ordering (partials written and read at device scope, the
 * flag stored after they complete); atomic adds fp32 into a zeroed fp32
 * output; workspace adds
 * fp32 into zeroed scratch followed by a second-stage reduce.
 *
 * Status codes follow the single-problem ABI of the stream-K GEMM bridge
 * (composable_kernel commit "feat(ck-tile): stream-K GEMM TE to dispatcher
 * bridge", Changes): 0 success, -1 a HIP error or C++ exception, -2 arguments
 * the engine does not support.  A -2 is decided on the host before anything
 * is enqueued, so outputs are untouched; skg_last_error() then names the
 * reason.  After a -1, work already enqueued may have run.
 *
 * Ownership: the caller owns every buffer (inputs, outputs, scales and the
 * workspace) and every stream; the library allocates no device memory in the
 * calls below.  Device pointers must be device memory of the current HIP
 * device.  Calls are asynchronous: 0 means "enqueued on the stream".
 *
 * Thread safety: all calls may be made from several host threads; the last
 * error string is per thread.  Two calls that share a workspace buffer must
 * not overlap in time on the device.
 */
#ifndef SKGEMM_H
#define SKGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKG_OK 0
#define SKG_ERR_HIP (-1)
#define SKG_ERR_UNSUPPORTED (-2)

/* Element types. */
enum skg_dtype {
  SKG_F16 = 0,     /* IEEE binary16 */
  SKG_BF16 = 1,    /* bfloat16 */
  SKG_F8E4M3 = 2,  /* OCP fp8 E4M3 (bias 7, max 448, no inf), the gfx950 fp8 */
  SKG_F32 = 3,     /* IEEE binary32 (outputs only) */
  SKG_F8E5M2 = 4   /* OCP bf8 E5M2 (bias 15, max 57344, inf and NaN: the upper
                      byte of an IEEE binary16), the gfx950 bf8 ("gemm_rowcolquant
                      dispatcher bridge" PR: fp8/bf8 rcr scope; OCP encoding on
                      gfx950 per its round-3 fixes) */
};

/* How scale_a / scale_b apply.  Row/column scaling is the "gemm_rowcolquant
 * dispatcher bridge" PR's own; per-tensor scaling is its sibling
 * "tensor_quant" (same PR, final description: one scalar scale for all of A
 * and one for all of B).
 *   SKG_SCALE_ROWCOL  scale_a holds M floats (one per row of A), scale_b N
 *                     floats (one per column of B);
 *   SKG_SCALE_TENSOR  scale_a and scale_b each hold one float for the whole
 *                     operand.
 * Either pointer may be NULL (scale 1) in both modes. */
enum skg_scale_mode {
  SKG_SCALE_ROWCOL = 0,
  SKG_SCALE_TENSOR = 1,
  /* SKG_SCALE_MX_E8M0  OCP Microscaling block scales (the MX / microscaling
   *                    variants named for the bquant bridge in the combined
   *                    follow-up of the "gemm_rowcolquant dispatcher bridge"
   *                    PR; the gfx950 scaled f8f6f4 MFMA of PR #13151's arch
   *                    table): scale_a points to M x K/32 and scale_b to
   *                    N x K/32 bytes, row-major, each an E8M0 code (value
   *                    2^(code-127), 255 = NaN) for one block of 32
   *                    consecutive K elements of a row of A or a column of B:
   *                    C[m][n] = round(sum_b 2^(sa[m][b]-127) 2^(sb[n][b]-127)
   *                    sum_{k in b} a(m,k) b(k,n)).  fp8 / bf8 inputs, the
   *                    128x128x128 or 256x256x128 tile, K a multiple of 128,
   *                    both pointers non-NULL and 16-byte aligned; no
   *                    further scale. */
  SKG_SCALE_MX_E8M0 = 2
};

/* Launch modes (PR #13151, Technical Details: Wgrad kernel, launch modes).
 *   SKG_MODE_DP         every tile is data-parallel, grid = tiles (the
 *                       comparator the stream-K launch is measured against);
 *   SKG_MODE_DP_SK      grid = stream-K CTAs (block ids 0..sk_ctas-1) then
 *                       one CTA per data-parallel tile;
 *   SKG_MODE_PERSISTENT grid = the pool; each CTA runs data-parallel tiles
 *                       b, b+grid, ... and its stream-K range: a first
 *                       segment that continues a tile begun by a lower CTA
 *                       (it hands its partial on, in a tree possibly after
 *                       folding higher positions) runs before the
 *                       data-parallel tiles, the segments it owns after
 *                       them (so their folds find the partials ready). */
enum skg_mode {
  SKG_MODE_DP = 0,
  SKG_MODE_DP_SK = 1,
  SKG_MODE_PERSISTENT = 2,
  /* SKG_MODE_SPLITK  comparator: every tile is cut into `ctas` equal K
   *                  slices (clamped to [1, iterations per tile]; ctas =
   *                  -1: as many as fill the default pool while every slice
   *                  keeps >= 8 MAC iterations), one CTA per slice; runs as
   *                  dp_sk with a pool of tiles x slices.  1 slice is plain
   *                  data-parallel. */
  SKG_MODE_SPLITK = 3,
  /* SKG_MODE_AUTO    the choice of the "auto" default of PR #13151 (commit
   *                  making stream-K the auto default, and its review
   *                  follow-up): dp_sk when the tiles leave a ragged wave
   *                  of the pool (tiles mod pool != 0, tiles < 2 x pool)
   *                  over a long reduction (>= 8 MAC iterations per tile)
   *                  and that partition has stream-K CTAs; split-K with
   *                  the default slice count otherwise.  skg_plan_* report
   *                  the launch it resolved to. */
  SKG_MODE_AUTO = 4
};

/* Fix-up of tiles shared by several stream-K CTAs (PR #13151, same section).
 *   LINEAR     deterministic: the owner folds the contributors in CTA order;
 *   TREE       deterministic: pairwise folds in ceil(log2 n) rounds;
 *   ATOMIC     fp32 atomics into the output, which must be fp32 (the call
 *              zeroes it first);
 *   WORKSPACE  fp32 atomics into scratch, then a second-stage kernel applies
 *              the epilogue and writes the output;
 *   SCATTER    deterministic reduce-scatter, not one of the page's four: for
 *              partitions that give every stream-K CTA one whole slice of
 *              one tile (sk_ctas = sk_tiles * S, S = iters_per_tile /
 *              iters_per_sk_cta, no extra iterations: split-K with S
 *              dividing the iterations, or any pool that divides them so).
 *              Every contributor publishes its fp32 partial; contributor k
 *              of a tile's S then sums the k-th of S equal parts of the tile
 *              over all S partials, in contributor order, and writes that
 *              part of the output: the additions and the epilogue of LINEAR
 *              in LINEAR's order, so the output is LINEAR's bit for bit for
 *              the same partition.  One round of hand-offs where linear
 *              takes S - 1 and tree ceil(log2 S); same workspace and the
 *              same residency rule as linear/tree.  Other partitions: -2.
 *              Never chosen by AUTO. */
enum skg_reduction {
  SKG_RED_LINEAR = 0,
  SKG_RED_TREE = 1,
  SKG_RED_ATOMIC = 2,
  SKG_RED_WORKSPACE = 3,
  SKG_RED_AUTO = 4, /* resolves to WORKSPACE: it never waits, so it takes the
                       occupancy-sized pool (same commit as SKG_MODE_AUTO) */
  SKG_RED_SCATTER = 5
};

/* Which stream-K CTA each block runs (the dispatch order of the partition's
 * CTAs; the partition itself is the same).  Workgroups go to the 8 XCDs of
 * gfx950 round robin, block i to XCD i mod 8, and each XCD has its own L2.
 *   SKG_SK_ORDER_AUTO   KMAJOR for wgrad (so XCD where the slices are not
 *                       whole), BLOCK for GEMM (measured: wgrad's stream-K
 *                       CTAs share the dY and X rows of a k range, GEMM's
 *                       neighbouring CTAs do not share lines);
 *   SKG_SK_ORDER_BLOCK  block b runs stream-K CTA b;
 *   SKG_SK_ORDER_XCD    the stream-K CTAs are dealt to the XCDs in contiguous
 *                       runs: block b runs CTA x*q + min(x, r) + b/8 with
 *                       x = b mod 8, q = sk_ctas / 8, r = sk_ctas mod 8, so
 *                       that CTAs sharing a tile, and neighbouring tiles,
 *                       share one L2;
 *   SKG_SK_ORDER_KMAJOR for a partition that gives every stream-K CTA one
 *                       whole slice of one tile (sk_ctas = sk_tiles * S
 *                       with S = iters_per_tile / iters_per_sk_cta and no
 *                       extra iterations, as split-K gives): the XCD runs
 *                       above are taken over the (slice, tile) pairs in
 *                       slice-major order, so block b runs CTA t*S + s for
 *                       the pair number c = x*q + min(x, r) + b/8, slice
 *                       s = c / sk_tiles, tile t = c mod sk_tiles.  The CTAs
 *                       running one k range of different tiles then share
 *                       an L2 and read the same rows of the operand that
 *                       does not depend on the tile's columns (dY for wgrad,
 *                       A for GEMM) at about the same time.  Any other
 *                       partition runs in XCD order; the plan reports the
 *                       order that runs.
 * The chiplet swizzle the pages reject with stream-K (PR #13151,
 * Constraints) remaps tiles; this remaps only whole stream-K ranges.
 * Waits still target higher CTA ids and all stream-K CTAs are co-resident,
 * so every wait ends in either order. */
enum skg_sk_order {
  SKG_SK_ORDER_AUTO = 0,
  SKG_SK_ORDER_BLOCK = 1,
  SKG_SK_ORDER_XCD = 2,
  SKG_SK_ORDER_KMAJOR = 3
};

/* Compiled tile instances.  TM x TN x TK in elements; each instance exists
 * for the operations and input types skg_tile_info reports. */
enum skg_tile {
  SKG_TILE_128x128x32 = 0,   /* f16/bf16 GEMM and wgrad, 4 waves */
  SKG_TILE_256x256x64 = 1,   /* f16/bf16 GEMM and wgrad, 4 waves */
  SKG_TILE_256x256x128 = 2,  /* fp8 GEMM (also with MX block scales), 4 waves */
  SKG_TILE_32x64x64 = 3,     /* f16/bf16 wgrad (small per-group M), 4 waves */
  SKG_TILE_128x128x64 = 4,   /* f16/bf16 GEMM and wgrad, 4 waves */
  SKG_TILE_256x128x64 = 5,   /* f16/bf16 GEMM and wgrad, 4 waves */
  SKG_TILE_128x128x128 = 6,  /* fp8 GEMM (also with MX block scales), 4 waves */
  SKG_TILE_64x144x32 = 7,    /* f16/bf16 grouped wgrad, block-diagonal: four whole
                                groups of 16 input and 16 output channels per
                                tile (GEMM-M = 64 output channels, GEMM-N = 9
                                filter taps x 16 channels), 4 waves */
  SKG_TILE_128x64x32 = 8,    /* f16/bf16 grouped forward conv and dgrad,
                                block-diagonal: 128 pixels x four whole groups
                                of 16 input and 16 output channels (GEMM-N =
                                64 channels), two filter taps per MAC
                                iteration, 4 waves */
  SKG_TILE_COUNT = 9
};

enum skg_op { SKG_OP_GEMM = 0, SKG_OP_WGRAD = 1, SKG_OP_FWD = 2, SKG_OP_DGRAD = 3 };

typedef struct skg_tile_info {
  int32_t tm, tn, tk;      /* tile in elements */
  int32_t n_waves;         /* wave64s per CTA (one flag per CTA and wave) */
  int32_t gemm_dtypes;     /* bit mask of 1 << skg_dtype accepted for GEMM A/B */
  int32_t wgrad_dtypes;    /* bit mask accepted for wgrad X/dY (0: no wgrad) */
  int32_t conv_dtypes;     /* bit mask accepted for forward conv and dgrad (0: none) */
  int32_t group_block;     /* block-diagonal wgrad tile: whole groups per tile
                              (each of 16 input and 16 output channels); 0:
                              dense tile, counted per group */
} skg_tile_info_t;

/* GEMM problem.  A is M x K row-major with leading dimension lda (elements),
 * B is K x N column-major (column n is K contiguous elements at B + n*ldb),
 * C is M x N row-major with leading dimension ldc.  scale_a (M floats) and
 * scale_b (N floats; one float each with SKG_SCALE_TENSOR) are optional
 * (NULL means 1.0); the epilogue computes
 * C[m][n] = round_to_nearest_even((acc * scale_a[m]) * scale_b[n]) in fp32
 * ("gemm_rowcolquant dispatcher bridge" PR, final description: scales applied
 * in the epilogue, fp32 accumulator narrowed only there).
 * Alignment: A, B, C 16-byte aligned; lda, ldb multiples of 16 bytes; K a
 * multiple of 16 bytes of input type; ldc a multiple of 16 bytes; lda, ldb
 * >= K and ldc >= N (else -2).  Only the first K elements of each A row and
 * B column are read, and only the M x N elements of C are written: padding
 * columns of C keep what they held. */
typedef struct skg_gemm_args {
  int64_t M, N, K;
  int32_t dtype_ab;        /* SKG_F16, SKG_BF16, SKG_F8E4M3 or SKG_F8E5M2 */
  int32_t dtype_c;         /* SKG_F16, SKG_BF16 or SKG_F32 */
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  void* C;
  int64_t ldc;
  const float* scale_a;    /* device pointer (16-byte aligned) or NULL; with
                              SKG_SCALE_MX_E8M0 the E8M0 byte array */
  const float* scale_b;    /* likewise */
  int32_t tile_id;         /* enum skg_tile */
  int32_t mode;            /* enum skg_mode */
  int32_t reduction;       /* enum skg_reduction */
  int32_t ctas;            /* stream-K pool (split-K: slices per tile); -1 = default;
                              0 or < -1 rejected */
  int32_t scale_mode;      /* enum skg_scale_mode */
  int32_t sk_order;        /* enum skg_sk_order */
} skg_gemm_args_t;

/* wgrad problem (PR #13151, Motivation and Technical Details).  X is the
 * forward input, NHWC (n, h, w, c); dY the output gradient, NHWC with
 * Ho = (h + 2*pad_h - r)/stride_h + 1 and Wo likewise (dilation 1); dW the
 * filter gradient, fp32, K x R x S x (C/groups) row-major.  Group g maps input
 * channels [g*C/groups, (g+1)*C/groups) to output channels
 * [g*K/groups, (g+1)*K/groups).  C/groups must be a multiple of 8 and
 * K/groups a multiple of 8; X, dY, dW 16-byte aligned.
 * Groups fold into GEMM-M (PR #13151, the wgrad port commit: GEMM-M = K).
 * Dense tiles are counted per group (groups * ceil(Kpg/TM) M tiles, so a
 * tile never spans two groups).  The block-diagonal tile SKG_TILE_64x144x32
 * needs C/groups == K/groups == 16; it holds four consecutive groups
 * (ceil(groups/4) M tiles, the last one possibly with fewer groups), and
 * each row's 144 columns are its own group's (tap, channel) entries, i.e.
 * ceil(R*S/9) N tiles of nine taps. */
typedef struct skg_wgrad_args {
  int32_t n, h, w, c, k, r, s;
  int32_t stride_h, stride_w, pad_h, pad_w, groups;
  int32_t dtype;           /* SKG_F16 or SKG_BF16 (X and dY) */
  const void* x;
  const void* dy;
  float* dw;
  int32_t tile_id, mode, reduction, ctas;
  int32_t sk_order;        /* enum skg_sk_order */
} skg_wgrad_args_t;

/* Forward convolution and input gradient (dgrad) as implicit GEMMs on the
 * same engine (PR #13151: the "docs" commit points the forward-convolution
 * future-work note at the stream-K port; review items 2-3 ask for forward
 * convolution on the family-agnostic partitioner).  Layouts as for wgrad:
 * NHWC activations, KRSC filter W (K x R x S x C/groups, the filter that
 * skg_run_wgrad differentiates), Ho = (h + 2*pad_h - r)/stride_h + 1,
 * dilation 1, group g maps input channels [g*C/groups, (g+1)*C/groups) to
 * output channels [g*K/groups, (g+1)*K/groups).
 *   forward  act = X (n,h,w,c), out = Y (n,Ho,Wo,k):
 *            Y[n][ho][wo][k] = sum_{r,s,c'} X[n][ho*sh-ph+r][wo*sw-pw+s][g*Cpg+c'] W[k][r][s][c']
 *            GEMM M = n*Ho*Wo, N = K/groups per group, reduction R*S*Cpg;
 *   dgrad    act = dY (n,Ho,Wo,k), out = dX (n,h,w,c): the adjoint of the
 *            forward map in X; GEMM M = n*h*w, N = C/groups per group,
 *            reduction R*S*Kpg.  Its run call first writes the filter
 *            transposed per group into the workspace (plan.aux_bytes), so
 *            both operands are contiguous along the reduction; with a stride
 *            above 1 the taps that reach no output pixel are multiplied as
 *            zeros (the MAC iterations are those of the stride-1 problem).
 * act and filt have type dtype (f16 or bf16); out has dtype_out (f16, bf16,
 * or f32, which the atomic reduction needs).  Channels per group (C/groups
 * and K/groups) must be multiples of 8; act, filt, out 16-byte aligned.  The
 * tiles are those whose skg_tile_info.conv_dtypes is non-zero.  Dense tiles
 * are counted per group along GEMM-N (groups * ceil(N per group / TN)); the
 * block-diagonal tile SKG_TILE_128x64x32 needs C/groups == K/groups == 16
 * and holds four consecutive groups (ceil(groups/4) N tiles), with a
 * reduction of R*S*16 per group (ceil(R*S/2) MAC iterations of two taps). */
typedef struct skg_conv_args {
  int32_t n, h, w, c, k, r, s;
  int32_t stride_h, stride_w, pad_h, pad_w, groups;
  int32_t dtype;           /* SKG_F16 or SKG_BF16 (act and filt) */
  int32_t dtype_out;       /* SKG_F16, SKG_BF16 or SKG_F32 */
  const void* act;         /* forward: X; dgrad: dY */
  const void* filt;        /* W, K x R x S x C/groups */
  void* out;               /* forward: Y; dgrad: dX */
  int32_t tile_id, mode, reduction, ctas;
  int32_t sk_order;        /* enum skg_sk_order */
} skg_conv_args_t;

/* Resolved launch plan, returned by value so that no derived quantity is
 * recomputed elsewhere with different rounding (PR #13151, commit adding the
 * iteration partitioner).  Iterations are MAC iterations: one TM x TN x TK
 * block of one output tile. */
typedef struct skg_plan {
  int32_t tm, tn, tk, n_waves;
  int32_t mode, reduction;
  int64_t tiles_m, tiles_n, tiles;
  int64_t iters_per_tile;
  int64_t pool;
  int64_t dp_tiles, sk_tiles, sk_ctas, sk_iters;
  int64_t iters_per_sk_cta;  /* clamped to >= 1, also for all-DP plans */
  int64_t extra_iters;       /* the first extra_iters stream-K CTAs run one more */
  int64_t grid;
  int64_t max_contrib;       /* most CTAs sharing one tile (1 when all-DP) */
  int64_t linear_partners;   /* max_contrib - 1 */
  int64_t tree_rounds;       /* ceil(log2(max_contrib)) */
  int64_t flags_bytes;       /* 4 * sk_ctas * n_waves rounded up to 256 (linear/tree) */
  int64_t partials_bytes;    /* sk_ctas * TM * TN * 4 (linear/tree) */
  int64_t workspace_bytes;   /* bytes the caller must pass as ws */
  int32_t requested_mode;    /* the mode asked for; `mode` is what runs */
  int32_t slices;            /* split-K slices per tile (1 unless split-K) */
  int32_t sk_order;          /* the order that runs: BLOCK, XCD or KMAJOR */
  int64_t aux_bytes;         /* workspace after the fix-up region that the op
                                itself uses (dgrad: the transposed filter);
                                included in workspace_bytes */
} skg_plan_t;

/* Reason for the last non-zero status on this thread ("" if none).  The
 * pointer stays valid until the next call on the same thread.  The reasons
 * are fixed strings per cause, as the wgrad launcher's rejections are on
 * PR #13151 (Technical Details: Constraints, the validator returning a
 * reason string for every rejected shape) and as the stream-K GEMM bridge
 * reports why a problem is unsupported (composable_kernel commit
 * "feat(ck-tile): stream-K GEMM TE to dispatcher bridge", Changes). */
const char* skg_last_error(void);

/* Tile instance table.  -2 for an unknown tile id. */
int skg_tile_info(int32_t tile_id, skg_tile_info_t* out);

/* Default pool for ctas = -1 (PR #13151, commits sizing the default pool):
 * one CTA per CU for linear/tree, whose CTAs wait on later CTAs; four per CU
 * for atomic/workspace, which never wait; never more per CU than
 * resident_per_cu.  Pure host function.  -2 on an unknown reduction or
 * non-positive counts. */
int skg_default_pool(int32_t reduction, int32_t num_cus, int32_t resident_per_cu,
                     int32_t* out);

/* Compute units of the current device and how many CTAs of the given kernel
 * instance stay resident per CU.  -1 if no HIP device is usable, -2 for an
 * unknown instance or a device that is not gfx950. */
int skg_device_info(int32_t op, int32_t tile_id, int32_t dtype_ab,
                    int32_t* num_cus, int32_t* resident_per_cu);

/* Plans.  Pure host functions except for ctas = -1, which asks the current
 * device for its CU count (skg_device_info).  Pointers in args are ignored.
 * 0, -1 (device query failed) or -2 (arguments unsupported, reason in
 * skg_last_error). */
int skg_plan_gemm(const skg_gemm_args_t* args, skg_plan_t* out);
int skg_plan_wgrad(const skg_wgrad_args_t* args, skg_plan_t* out);
int skg_plan_fwd(const skg_conv_args_t* args, skg_plan_t* out);
int skg_plan_dgrad(const skg_conv_args_t* args, skg_plan_t* out);

/* Bytes of workspace the run call needs for these arguments: the plan's
 * workspace_bytes (PR #13151, Technical Details: Partitioner -- the flag
 * table of one int32 per stream-K CTA and wave, rounded up to 256 bytes,
 * then one fp32 partial tile per stream-K CTA for linear/tree; one fp32
 * tile per stream-K tile for workspace; nothing for atomic or a plan
 * without stream-K CTAs).  Same status codes as skg_plan_*. */
int skg_gemm_workspace_bytes(const skg_gemm_args_t* args, size_t* out);
int skg_wgrad_workspace_bytes(const skg_wgrad_args_t* args, size_t* out);

/* Run (composable_kernel commit "feat(ck-tile): stream-K GEMM TE to
 * dispatcher bridge", Changes: one problem per call, 0 / -1 / -2; PR #13151,
 * Technical Details: Wgrad kernel, for the launch modes, the resets and the
 * four reductions).
 * ws must point to at least plan.workspace_bytes of device memory
 * (may be NULL when that is 0); the call resets on the stream whatever the
 * reduction accumulates into: the flags (linear/tree), the scratch
 * (workspace) or C itself (atomic).  Partials and, for linear/tree, C are
 * never pre-zeroed.  Linear and tree results are bit-identical from launch to
 * launch.  For linear/tree the stream-K CTAs must all be resident at once, so
 * a pool larger than the device's resident capacity for the instance is
 * rejected with -2.  stream is a hipStream_t (NULL: the null stream). */
int skg_run_gemm(const skg_gemm_args_t* args, void* ws, size_t ws_bytes, void* stream);
int skg_run_wgrad(const skg_wgrad_args_t* args, void* ws, size_t ws_bytes, void* stream);
int skg_run_fwd(const skg_conv_args_t* args, void* ws, size_t ws_bytes, void* stream);
int skg_run_dgrad(const skg_conv_args_t* args, void* ws, size_t ws_bytes, void* stream);

/* Allocation-free wgrad, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, plan and results as skg_run_wgrad, but the
 * flags, partials or scratch live in one library-owned device array of
 * SKG_STATIC_SCRATCH_BYTES per device (allocated with the library's code
 * object on that device and held until the process ends), and the resets are
 * done by a small fill kernel instead of hipMemsetAsync.  The call itself
 * allocates nothing.  A plan whose workspace_bytes exceeds the array is
 * rejected with -2 (the reason names both sizes); e.g. the 256x128x64 tile
 * on N=32 56x56 C=K=256 3x3 fits with every reduction at a pool of 256.
 * Every call on one device shares that device's array and leaves its
 * contents behind: two calls that overlap in time on one device (different
 * streams, or different host threads) race and give wrong results; calls
 * on one stream are ordered and safe.  Status codes as skg_run_wgrad. */
#define SKG_STATIC_SCRATCH_BYTES (33u << 20)
int skg_run_wgrad_static(const skg_wgrad_args_t* args, void* stream);

/* Hand-off waits that gave up.  A linear/tree wait polls its partner's flag
 * a bounded number of times (PR #13151, review items: forward progress rests
 * on in-order dispatch, which the hardware does not promise); a wait that
 * gives up counts one event per wave here and the fold goes on with whatever
 * the partner's partial buffer holds, so the values of that tile are then
 * unspecified: a caller that cannot rule out a pool larger than what stays
 * resident (another process taking CUs) checks this count.  It is summed
 * over every kernel instance since the last reset; with reset != 0 the
 * counters are zeroed after reading.  Call only while no run call's kernels
 * are executing (after a device or stream synchronisation).  0, or -1 if
 * the counters cannot be read.
 *
 * Fault injection for tests of these paths (environment, read by every run
 * call): SKG_FAULT=launch makes a run call return -1 where it would launch
 * the stream-K kernel, after its resets are enqueued; SKG_FAULT=handoff
 * launches it with stream-K CTAs that store their partials but never raise
 * their flags and a spin limit of 64 polls, so every hand-off wait gives up
 * quickly and the kernel still ends. */
int skg_fixup_timeouts(uint32_t* count, int32_t reset);

/* Timing hook for measurement: while set on the calling thread, every run
 * call records `start` (a hipEvent_t) on its stream immediately before the
 * stream-K kernel and `stop` immediately after it -- after the resets and
 * before any second stage -- so the pair times that kernel alone.  Both NULL
 * clears the hook; passing only one is -2.  The events stay owned by the
 * caller. */
int skg_profile_events(void* start, void* stop);

#ifdef __cplusplus
}
#endif

#endif /* SKGEMM_H */
