/*
 * sdt.h -- C ABI of the MI355X (gfx950) fp16 GEMM and M=1 decode GEMV.
 *
 * The operation is the fp16 matrix product of "Beating hipBLASLt on a Gaming
 * GPU" (section "The result": square fp16 GEMM) and of the mojo-baro project
 * page (section "Four rounds on the decode shape": the M=1, K=4096, N=12288
 * skinny product whose weights stream from HBM), in the transposed-B form
 * C = A @ B_T.T benchmarked by the FlyDSL pull request "Speed up the RDNA3
 * GEMM up to 1.85x by choosing the tile from the shape" (Performance).
 *
 * Layouts (all strides in elements, taken from the caller, never assumed
 * tight -- FlyDSL PR, Changes: caller-supplied lda/ldb/ldc):
 *   A(m,k) = A[m*lda + k]   (M x K, row-major)
 *   B(k,n) = B[n*ldb + k]   ("K-major": K contiguous, N rows of length ldb)
 *   C(m,n) = C[m*ldc + n]   (M x N, row-major)
 * Elements are IEEE binary16 bit patterns.  Products are accumulated in fp32
 * and the result is rounded to fp16 with round-to-nearest-even (overflow to
 * +-inf).  C is overwritten (no alpha/beta).
 *
 * Ownership and execution: every pointer is a device pointer owned by the
 * caller and must stay valid until the enqueued work completes; C must not
 * alias A or B.  Calls enqueue on `stream` (a hipStream_t passed as void*;
 * NULL is the default stream) of the calling thread's current HIP device and
 * return without synchronising.  The library allocates no memory per call,
 * never prints, aborts or exits, and is safe to call from several threads.
 *
 * Errors: every call returns an sdt_status.  On any error nothing is
 * enqueued.  SDT_ERR_HIP keeps the HIP error code for sdt_last_hip_error().
 */
#ifndef SDT_H
#define SDT_H

#include <stdint.h>

/* Version of the structures and signatures below; bumped whenever sdt_tile,
 * sdt_launch or an entry point's arguments change, or entry points are added
 * (4: the off-ladder rungs 5-7, the [K][N] workspace entry points and
 * sdt_stream_read_runs; 5: sdt_mfma_ceiling, and loader waves: the `loaders`
 * field of sdt_tile and sdt_launch).
 * sdt_abi_version() reports the version the library was built with: a caller
 * compiled against another header must not pass these structures to it. */
#define SDT_ABI_VERSION 5

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sdt_status {
    SDT_OK = 0,
    SDT_ERR_INVALID_ARG = 1,  /* negative size, null pointer with work to do,
                                 leading dimension smaller than the row */
    SDT_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels handle:
                                 misaligned pointer or stride, size limits */
    SDT_ERR_HIP = 3           /* the HIP runtime refused the launch */
} sdt_status;

/* One rung of the tile ladder: a compile-time instantiation of the GEMM
 * kernel (bm x bn output block per workgroup, bk = k-tile depth, waves_m x
 * waves_n wavefronts of 64 lanes), after "Beating hipBLASLt on a Gaming GPU",
 * section "The part that actually mattered" (tile shape as a compile-time
 * kernel parameter, each with its own warp layout). */
typedef struct sdt_tile {
    int id;          /* rung index: 0-4 the ladder, largest tile first (256 x 256,
                        256 x 128, 128 x 128, 128 x 64, 64 x 64); 5, 6 and 7
                        the off-ladder 96 x 96, 192 x 192 and 160 x 160
                        tiles (see sdt_pick_tile) */
    int bm, bn, bk;
    int waves_m, waves_n;
    int threads;     /* 64 * waves_m * waves_n * kgroups, twice that with loaders */
    int stages;      /* LDS stages: the global prefetch runs stages - 1 k-tiles deep
                        (sdt_pick_tile: the count a launch of that shape uses;
                        sdt_tile_info: the rung's deep pipeline).  On rung 0
                        the deep count (3) is the ping-pong kernel: two groups
                        of 4 waves one phase apart, A in 2 stages, B in 3.
                        On rungs 1-4 (256 x 128 down to 64 x 64) the deep
                        count with one k-group runs v_mfma_f32_16x16x32 (two
                        32-deep sub-steps per k-tile), and so does every
                        pipeline of rungs 5-7 (96 x 96 with 48 x 48 per wave,
                        192 x 192 with 96 x 48, 160 x 160 with 80 x 80);
                        every other launch runs v_mfma_f32_32x32x16.  The automatic plan takes the
                        long count (long_stages) in place of the deep one on a
                        rung that has it when the launch runs two k-groups and
                        K holds at least 12 full k-tiles */
    int lds_bytes;   /* stages x (bm + bn) x bk fp16; rung 0 deep:
                        (2 bm + 3 bn) x bk fp16 = 160 KB */
    int kgroups;     /* groups of waves splitting each k-tile's four 16-deep
                        sub-steps (1 or 2; sdt_tile_info: the most the rung is
                        built with) */
    int stagger;     /* 1: the automatic plan visits the k-tiles staggered,
                        (workgroup + i) & (k-tiles - 1) (sdt_tile_info: 0) */
    int long_stages; /* a deeper pipeline for long k-loops (4 on the 128 x 64
                        and 64 x 64 rungs), 0 if the rung has none */
    int splits;      /* workgroups each output tile's k-loop is split over
                        (1: none).  Only the workspace entry points split */
    int split_algo;  /* splits > 1: how the fp32 partial sums are reduced, in
                        split order: 0 by a second kernel, 1 by the last
                        workgroup of each tile in the same kernel */
    int persistent;  /* 0: one workgroup per tile; P > 0: P workgroups loop
                        over the tiles (ping-pong kernel only) */
    int ksplit;      /* 1: the rung is built to split K across workgroups */
    int loaders;     /* 1: a loader wave beside each compute wave issues every
                        global -> LDS load, so that the compute waves issue only
                        fragment reads and MFMAs (the deep one-k-group pipeline
                        of rungs 1, 2 and 4, 256 x 128, 128 x 128 and 64 x 64,
                        without a k-split; the automatic plan from 12 full k-tiles;
                        sdt_tile_info: 1 where the rung is built with them) */
} sdt_tile;

/* A launch configuration; -1 in a field = the automatic choice. */
typedef struct sdt_launch {
    int tile_id;     /* ladder rung */
    int stages;      /* 2, the rung's deep count (sdt_tile_info().stages) or
                        its long count (sdt_tile_info().long_stages, if any) */
    int kgroups;     /* 1, or 2 on rungs built with two (needs the deep or long
                        count) */
    int stagger;     /* 0 off, 1 on (power-of-two full k-tile count only) */
    int splits;      /* 1 none; s in [2, 64] on a ksplit rung: K split over s
                        workgroups per tile (at most one per full k-tile, no
                        stagger), needs the workspace sdt_launch_workspace_size
                        reports */
    int split_algo;  /* 0 a second kernel sums the partials, 1 the last
                        workgroup of each tile does */
    int persistent;  /* 0 off; P in [1, tiles]: the ping-pong kernel (rung 0's
                        deep pipeline) runs P workgroups, workgroup w taking
                        tiles w, w + P, w + 2P, ... (the FlyDSL PR, Changes:
                        persistent workgroups, where only 0 or the tile count
                        is accepted; any P in between is accepted here) */
    int loaders;     /* 0 off, 1 on: loader waves issue the global loads (rungs
                        1, 2 and 4 with their deep count, one k-group, no k-split) */
} sdt_launch;

/* ---- main entry points ---------------------------------------------------- */

/* C = A.B for M x N x K.
 * Requirements: M, N, K >= 0; lda >= K, ldb >= K, ldc >= N (else
 * SDT_ERR_INVALID_ARG); A, B, C 16-byte aligned and lda, ldb, ldc multiples of
 * 8 elements, lda and ldb below 2^22, M and N at most 2^31 - 1 (else
 * SDT_ERR_UNSUPPORTED).  Any M, N, K
 * within those limits is computed exactly as defined (ragged edges are
 * masked).  M == 0 or N == 0 is a no-op; K == 0 writes zeros (the empty sum).
 * M == 1 runs the streaming decode kernel of gemv_f16_m1 (same result
 * definition).  The tile is chosen by sdt_pick_tile from the device's CU
 * count.  The k-loop runs in plain k order except where the plan staggers it
 * (FlyDSL PR, Changes: workgroup w starts at k-tile w and wraps): on ladder
 * rungs 1-4 (not the ping-pong kernel), with a power-of-two count of at least 16
 * full k-tiles, and A and B together within 16 MiB (2*K*(M+N) bytes), where
 * it measured 2-5% faster on MI355X; larger operands lose up to 49% with it
 * (sdt_plan_tile reports the choice). */
int gemm_f16(int64_t M, int64_t N, int64_t K,
             const void* A, int64_t lda,
             const void* B, int64_t ldb,
             void* C, int64_t ldc, void* stream);

/* gemm_f16 with a workspace, which lets the plan split the k-loop across
 * workgroups ("Iteratively Tuning hipBLASLt TensileLite Kernels", The Six
 * Rounds, 2: splitting K is how shapes that cannot fill the device get work).
 * When the grid of gemm_f16's tile leaves CUs idle and the k-loop is long
 * (each split keeps at least 16 full k-tiles: on MI355X shorter loops ran
 * slower split), each output tile's k-tiles are divided into `splits`
 * contiguous runs, one workgroup each, with splits = min(CUs / tiles,
 * full k-tiles / 16, 16); their fp32 partial sums go to the workspace and a
 * second kernel adds them in split order, ((P_0 + P_1) + P_2) + ..., before
 * the single rounding to fp16, so the result is deterministic (no atomics on
 * the data).  Example: 256 x 256 x 16384 runs 16 splits of 64 x 64 tiles.
 * workspace: device memory owned by the caller, 16-byte aligned, at least
 * sdt_gemm_workspace_size(M, N, K, 0) bytes for the split plan (smaller, or
 * NULL with 0: the call runs gemm_f16's plan, unsplit, and touches no
 * workspace).  Layout: the first 64 KiB hold arrival counters (one int per
 * output tile, so a split launch has at most 16384 tiles),
 * the fp32 partial sums follow.  The counter area must be zero before the
 * first call that uses the workspace (sdt_workspace_init); every call leaves
 * it zero again, whatever its shape.  One workspace serves one call at a
 * time: calls that share it must be ordered on one stream (concurrent calls
 * on other streams need their own).
 * Everything else as gemm_f16 (same requirements, statuses and
 * degenerate-size behaviour; M == 1 runs the decode GEMV). */
int gemm_f16_ws(int64_t M, int64_t N, int64_t K,
                const void* A, int64_t lda,
                const void* B, int64_t ldb,
                void* C, int64_t ldc,
                void* workspace, int64_t workspace_bytes, void* stream);

/* gemm_f16_ws for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same plan and the same result bits as gemm_f16_ws with a workspace of
 * sdt_gemm_workspace_size bytes, with the k-split workspace taken from a
 * library-owned array of 16 MiB + 64 KiB per device (static device memory,
 * held until the process ends; its address is looked up, and its counter
 * area cleared by a kernel on `stream`, on the first call on each device).
 * Calls no allocating routine.  A product whose plan needs more workspace
 * than that array holds (only on a device with more than 256 CUs) returns
 * SDT_ERR_UNSUPPORTED and enqueues nothing.  All calls on one device share
 * the array: calls that overlap on one GPU (other streams, concurrent graph
 * replays) race and must be ordered by the caller.  Otherwise as gemm_f16. */
int gemm_f16_noalloc(int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda,
                     const void* B, int64_t ldb,
                     void* C, int64_t ldc, void* stream);

/* Bytes of workspace gemm_f16_ws's automatic plan uses for this product on a
 * device with num_cu compute units (num_cu <= 0 reads the current device);
 * 0 when it does not split.  Negative sizes, or M, N or K past 2^31 - 1: -1. */
int64_t sdt_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int num_cu);

/* Bytes of workspace a launch configuration (as gemm_f16_cfg takes it, every
 * field given) needs for an M x N product: 0 without a split; -1 for an
 * invalid configuration. */
int64_t sdt_launch_workspace_size(int64_t M, int64_t N, int64_t K, const sdt_launch* cfg);

/* Enqueue on `stream` the zero fill of a workspace's `bytes` bytes (a kernel,
 * so it may be captured into a graph).  workspace 16-byte aligned, bytes a
 * multiple of 4.  SDT_OK, SDT_ERR_INVALID_ARG, SDT_ERR_UNSUPPORTED or
 * SDT_ERR_HIP. */
int sdt_workspace_init(void* workspace, int64_t bytes, void* stream);

/* y(n) = sum_k x(k) * B(k,n), n < N: the M=1 decode product (mojo-baro page,
 * "Four rounds on the decode shape"), with B stored K-major as above (column n
 * of the math B is the contiguous run B[n*ldb .. n*ldb+K-1]); x holds K fp16
 * values, y receives N fp16 values.  Requirements as for gemm_f16 with M = 1
 * (x, B 16-byte aligned, ldb % 8 == 0).  N == 0 is a no-op, K == 0 writes
 * zeros. */
int gemv_f16_m1(int64_t N, int64_t K, const void* x,
                const void* B, int64_t ldb, void* y, void* stream);

/* y(n) = sum_k x(k) * B[k*ldb + n], n < N: the same M=1 decode product with
 * the weights stored as K rows of ldb >= N elements, the N of one row
 * contiguous (the "B-layout" of the mojo-baro page, "Four rounds on the decode
 * shape", where each thread owns contiguous columns).  x holds K fp16, y
 * receives N fp16 (round-to-nearest-even from an fp32 sum).  Requirements:
 * N, K >= 0 and ldb >= N when K > 0 (else SDT_ERR_INVALID_ARG); x and B
 * 16-byte aligned, ldb % 8 == 0 when K > 1, y 2-byte aligned (else
 * SDT_ERR_UNSUPPORTED).  N == 0 is a no-op, K == 0 writes zeros.  Deterministic:
 * the partial sums over K are combined in a fixed order; no workspace. */
int gemv_f16_m1_kn(int64_t N, int64_t K, const void* x,
                   const void* B, int64_t ldb, void* y, void* stream);

/* gemv_f16_m1_kn with a workspace, which lets the product split K across
 * workgroups: bands of 256 columns (512-byte runs of every weight row, where
 * the one-launch kernel reads 128-byte runs: on MI355X such runs stream at
 * most 5.46 TB/s, 512-byte ones 6.29) with K cut into `splits` ranges so that
 * about 768 workgroups stream at once; each writes its fp32 column sums to
 * the workspace and a second kernel adds the splits in split order, then
 * rounds once.  Deterministic; the bits differ from gemv_f16_m1_kn's (another
 * summation order), within the same error bound.  workspace: device memory
 * owned by the caller, 16-byte aligned, at least sdt_gemv_kn_workspace_size(N,
 * K) bytes for the split (smaller, or NULL with 0: the call runs
 * gemv_f16_m1_kn); needs no initialisation; one workspace serves one call at a
 * time (calls that share it must be ordered on one stream).  Errors as
 * gemv_f16_m1_kn, plus SDT_ERR_INVALID_ARG for workspace_bytes < 0 or a NULL
 * workspace with bytes > 0, SDT_ERR_UNSUPPORTED for a misaligned one. */
int gemv_f16_m1_kn_ws(int64_t N, int64_t K, const void* x, const void* B, int64_t ldb,
                      void* y, void* workspace, int64_t workspace_bytes, void* stream);

/* Bytes of workspace gemv_f16_m1_kn_ws splits with for an N x K product: 0
 * when it does not split (K < 16 or K > 2^30 - 1, N > 2^31 - 1, or a grid of
 * 768 band workgroups without a split); -1 for negative sizes.  Host-only. */
int64_t sdt_gemv_kn_workspace_size(int64_t N, int64_t K);

/* ---- bfloat16 variants ------------------------------------------------------
 * The same products with bfloat16 operands and output (1 sign, 8 exponent,
 * 7 fraction bits; fp32 accumulation on v_mfma_f32_32x32x16_bf16 /
 * v_dot2_f32_bf16; fp32 -> bf16 round-to-nearest-even).  The FlyDSL pull
 * request measures its square GEMMs in bf16 (Performance), and the mojo-baro
 * page's decode rounds run bf16 weight arms ("Four rounds on the decode
 * shape").  Same layouts, requirements, tile choice, statuses and
 * degenerate-size behaviour as the fp16 entry point of the same name;
 * gemm_bf16 with M == 1 runs gemv_bf16_m1. */
int gemm_bf16(int64_t M, int64_t N, int64_t K,
              const void* A, int64_t lda,
              const void* B, int64_t ldb,
              void* C, int64_t ldc, void* stream);
int gemm_bf16_ws(int64_t M, int64_t N, int64_t K,
                 const void* A, int64_t lda,
                 const void* B, int64_t ldb,
                 void* C, int64_t ldc,
                 void* workspace, int64_t workspace_bytes, void* stream);
int gemv_bf16_m1(int64_t N, int64_t K, const void* x,
                 const void* B, int64_t ldb, void* y, void* stream);
int gemv_bf16_m1_kn(int64_t N, int64_t K, const void* x,
                    const void* B, int64_t ldb, void* y, void* stream);
int gemv_bf16_m1_kn_ws(int64_t N, int64_t K, const void* x, const void* B, int64_t ldb,
                       void* y, void* workspace, int64_t workspace_bytes, void* stream);

/* ---- test / benchmark extras ---------------------------------------------- */

/* gemm_f16 with the launcher's choices forced.  tile_id: -1 = automatic,
 * else a ladder index (SDT_ERR_INVALID_ARG if out of range).  stagger: -1 =
 * what gemm_f16 does (the plan's choice), 0 = off, 1 = on (SDT_ERR_UNSUPPORTED
 * unless sdt_stagger_eligible(K)).  M == 1 is not rerouted to the GEMV here. */
int gemm_f16_ex(int64_t M, int64_t N, int64_t K,
                const void* A, int64_t lda,
                const void* B, int64_t ldb,
                void* C, int64_t ldc, void* stream,
                int tile_id, int stagger);

/* gemm_f16_ws / gemm_bf16_ws with any part of the launch configuration
 * forced (NULL cfg, an index out of range, a combination the library has no
 * kernel for, or a split whose workspace is missing or smaller than
 * sdt_launch_workspace_size: SDT_ERR_INVALID_ARG; a forced stagger on an
 * ineligible K: SDT_ERR_UNSUPPORTED).  splits == -1 lets the plan split when
 * the workspace allows, as gemm_f16_ws does.  M == 1 is not rerouted to the
 * GEMV here. */
int gemm_f16_cfg(int64_t M, int64_t N, int64_t K,
                 const void* A, int64_t lda,
                 const void* B, int64_t ldb,
                 void* C, int64_t ldc,
                 void* workspace, int64_t workspace_bytes, void* stream,
                 const sdt_launch* cfg);
int gemm_bf16_cfg(int64_t M, int64_t N, int64_t K,
                  const void* A, int64_t lda,
                  const void* B, int64_t ldb,
                  void* C, int64_t ldc,
                  void* workspace, int64_t workspace_bytes, void* stream,
                  const sdt_launch* cfg);

/* gemm_bf16 with the launcher's choices forced (as gemm_f16_ex). */
int gemm_bf16_ex(int64_t M, int64_t N, int64_t K,
                 const void* A, int64_t lda,
                 const void* B, int64_t ldb,
                 void* C, int64_t ldc, void* stream,
                 int tile_id, int stagger);

/* gemv_f16_m1 with the kernel instantiation forced: variant in
 * [0, sdt_gemv_num_variants()).  Variant 0, what gemv_f16_m1 uses: one column
 * per workgroup of four waves splitting K.  Variants 1-4: one wave streams 1,
 * 2, 4 or 8 whole columns (these four add in the same order and agree bit
 * for bit; variant 0 adds the same products in another order).  Same result
 * definition. */
int gemv_f16_m1_ex(int64_t N, int64_t K, const void* x,
                   const void* B, int64_t ldb, void* y, void* stream,
                   int variant);
int sdt_gemv_num_variants(void);

/* gemv_f16_m1_kn with the instantiation forced: variant in
 * [0, sdt_gemv_kn_num_variants()) selects the column band per workgroup and
 * the number of waves splitting K (variant 0 is what gemv_f16_m1_kn uses).
 * Same result definition; the combination order of partial sums differs. */
int gemv_f16_m1_kn_ex(int64_t N, int64_t K, const void* x,
                      const void* B, int64_t ldb, void* y, void* stream,
                      int variant);
int sdt_gemv_kn_num_variants(void);

/* Host-only: the tile the launcher would use for an M x N x K product on a
 * device with num_cu compute units (num_cu <= 0 reads the current device).
 * The rule compares the number of output blocks the grid produces with the
 * CU count ("Beating hipBLASLt on a Gaming GPU", "The part that actually
 * mattered"; ladder constants fitted on MI355X): the ladder's pick is
 * sdt_pick_rung over rungs 0-4 with rung r taken from
 * (bm/64)(bn/64)(num_cu/2 + 1) 64 x 64 blocks up (the last rung below that).
 * An off-ladder rung with a smaller tile replaces the pick when its grid has
 * more workgroups than the pick's, at most num_cu and at least 7/8 of num_cu
 * (the first such rung in id order), and, where the pick runs loader waves
 * (see sdt_tile.loaders), a tile of at most 2/3 of the pick's area: on MI355X
 * the 96 x 96 rung in place of 128 x 128 (e.g. 1536^3: 144 workgroups ->
 * 256), the 192 x 192 rung in place of 256 x 256 (e.g. 3072^3: 144 -> 256)
 * and the 160 x 160 rung in place of 256 x 128 on k-loops shorter than 12
 * k-tiles (e.g. 2560 x 2560 x 640: 200 -> 256).  Where the pick is rung 0 and
 * its grid has more than num_cu and at most 3/2 num_cu workgroups, rung 1
 * (256 x 128, with loader waves) replaces it on k-loops of at least 32
 * k-tiles (e.g. 4608^3: 324 ping-pong workgroups, two waves, against 648 of
 * 256 x 128 in three shorter ones), and where it has more than 2 num_cu and
 * at most 9/4 num_cu, on k-loops of at least 64 k-tiles (e.g. 6144^3).
 * Touches no device when num_cu > 0.  Returns SDT_OK, SDT_ERR_INVALID_ARG, or
 * SDT_ERR_UNSUPPORTED for M, N or K past 2^31 - 1. */
int sdt_pick_tile(int64_t M, int64_t N, int64_t K, int num_cu, sdt_tile* out);

/* Host-only: the plan gemm_f16_ws makes with a workspace of workspace_bytes
 * bytes (the k-split is taken only when it fits); otherwise as
 * sdt_pick_tile. */
int sdt_pick_tile_ws(int64_t M, int64_t N, int64_t K, int num_cu, int64_t workspace_bytes,
                     sdt_tile* out);

/* Host-only, the mechanism of the rule above: given `rungs` thresholds in
 * units of ref_bm x ref_bn output blocks (largest tile first, non-increasing),
 * returns the first rung r with ceil(M/ref_bm)*ceil(N/ref_bn) >=
 * min_blocks[r], or rungs-1 if none qualifies; -1 on invalid input (M or N
 * negative or past 2^31 - 1, a reference size or `rungs` not positive, NULL
 * thresholds). */
int sdt_pick_rung(int64_t M, int64_t N, int ref_bm, int ref_bn,
                  int rungs, const int64_t* min_blocks);

/* Host-only: number of rungs (the ladder's and the off-ladder ones), and
 * the description of rung tile_id (with its deep pipeline; long_stages names
 * its long one, if any). */
int sdt_num_tiles(void);
int sdt_tile_info(int tile_id, sdt_tile* out);

/* Host-only: how a launch of rung tile_id on an M x N x K product on num_cu
 * CUs (num_cu <= 0: 256) is configured (stages, kgroups, threads, LDS).
 * k-groups: 2 on rungs built with them by each rung's thresholds on the grid
 * and the k-loop (K in 64-deep k-tiles, at least 12): never on rungs 1 and 2
 * (their one-k-group pipeline runs loader waves); rung 3 with fewer than 3/4
 * of num_cu and at least 96 k-tiles; rung 4 with at most num_cu workgroups
 * and at least 40 k-tiles; else 1 (a k-split launch of gemm_f16_ws:
 * 2 whenever its grid of tiles x splits fits num_cu -- on rungs 1 and 2 with
 * fewer -- and each split runs at least 12 k-tiles).  Stages: the rung's deep
 * count, which with two k-groups becomes
 * the rung's long count (long_stages, the 128 x 64 and 64 x 64 rungs) once K
 * holds at least 12 full k-tiles; the 2-stage pipeline is never planned (it
 * lost with the operands in HBM and tied with them in L2).  Stagger: as
 * gemm_f16 describes.  SDT_OK, SDT_ERR_INVALID_ARG, or SDT_ERR_UNSUPPORTED for M,
 * N or K past 2^31 - 1. */
int sdt_plan_tile(int tile_id, int64_t M, int64_t N, int64_t K, int num_cu,
                  sdt_tile* out);

/* Host-only: 1 if the k-loop of a product with inner size K can be staggered,
 * else 0: the number of full 64-deep k-tiles floor(K/64) must be a power of
 * two, since the wrap-around is a mask (FlyDSL PR, Changes; the PR enables
 * the stagger exactly then).  On MI355X gemm_f16 staggers only the eligible
 * products gemm_f16 describes: with larger operands it loses up to 49%
 * (2048x2048x8192), since workgroups that share operand rows through one
 * XCD's L2 stop reading the same k-tile at the same time. */
int sdt_stagger_eligible(int64_t K);

/* Host-only: the k-tile visited at step i by workgroup wg when staggered:
 * (wg + i) & (nkt - 1); nkt must be a power of two (else -1). */
int64_t sdt_stagger_ktile(int64_t wg, int64_t i, int64_t nkt);

/* Measurement: enqueue an empty kernel (one workgroup of 64 lanes, no memory
 * access) on `stream`.  Timed back to back it gives the launch floor that the
 * smallest products are compared with (the pages report small shapes next to
 * such a floor).  Returns SDT_OK or SDT_ERR_HIP. */
int sdt_empty_kernel(void* stream);

/* Measurement: enqueue a read-only streaming kernel over `bytes` bytes of
 * device memory at `buf` (one wave per 8 KB run, eight non-temporal 16-byte
 * loads per lane: the access pattern of gemv_f16_m1, with no activations,
 * arithmetic or output).  Each 8 KB run is folded into one 32-bit word written
 * to out[run], so `out` (device, caller-owned) holds bytes / 8192 words; the
 * words have no meaning beyond keeping every load live.  Timed back to back
 * over the decode shape's rotating weight buffers it gives the streaming-read
 * ceiling the decode GEMV is reported against.  bytes == 0: SDT_OK, nothing
 * enqueued.  SDT_ERR_INVALID_ARG: bytes < 0 or a null pointer.
 * SDT_ERR_UNSUPPORTED: bytes not a multiple of 8192 (or more than 2^31 - 1
 * runs), buf not 16-byte aligned or out not 4-byte aligned.  SDT_ERR_HIP: the
 * launch failed. */
int sdt_stream_read(const void* buf, int64_t bytes, void* out, void* stream);

/* Measurement: enqueue a grid-stride read-only kernel over `bytes` bytes at
 * `buf`: `workgroups` workgroups of 256 threads, each pass reading 4 KB per
 * workgroup with four non-temporal 16-byte loads per lane, striding by the
 * whole grid (a plain bandwidth-test pattern, unlike either GEMV's).  Writes
 * one 32-bit word per workgroup to out[0 .. workgroups) (device,
 * caller-owned), with no meaning beyond keeping the loads live.  It gives a
 * streaming-read ceiling independent of the GEMV kernels' own access pattern.
 * bytes == 0: SDT_OK, nothing enqueued.  SDT_ERR_INVALID_ARG: bytes < 0, a
 * null pointer or workgroups <= 0.  SDT_ERR_UNSUPPORTED: bytes not a
 * multiple of 16, buf not 16-byte or out not 4-byte aligned.  SDT_ERR_HIP:
 * the launch failed. */
int sdt_stream_read_grid(const void* buf, int64_t bytes, void* out, int workgroups,
                         void* stream);

/* Measurement: enqueue a read-only kernel over `rows` rows of row_bytes bytes
 * at `buf`, read in runs of run_bytes contiguous bytes per row, the access
 * pattern of a [K][N] decode GEMV whose workgroups own column bands:
 * workgroup w (256 threads) reads band w % (row_bytes / run_bytes) of rows
 * [c * rows_per_wg, (c + 1) * rows_per_wg), c = w / (row_bytes / run_bytes),
 * with 16-byte non-temporal loads, 8 per lane in flight.  Grid: (row_bytes /
 * run_bytes) * (rows / rows_per_wg) workgroups, each writing one 32-bit word
 * (the XOR of every 32-bit word it read) to out[w].  rows == 0: SDT_OK,
 * nothing enqueued.  SDT_ERR_INVALID_ARG: negative rows, row_bytes <= 0, a
 * null pointer, run_bytes not 64, 128, 256, 512 or 1024, row_bytes not a
 * multiple of run_bytes, rows_per_wg not a positive multiple of 8 * 4096 /
 * run_bytes, or rows not a multiple of rows_per_wg.  SDT_ERR_UNSUPPORTED: buf
 * not 16-byte or out not 4-byte aligned, or a grid past 2^31 - 1.
 * SDT_ERR_HIP: the launch failed. */
int sdt_stream_read_runs(const void* buf, int64_t rows, int64_t row_bytes, int run_bytes,
                         int rows_per_wg, void* out, void* stream);

/* Host-only argument check used by gemv_f16_m1_kn before anything is
 * enqueued (the status it would return for these arguments). */
int sdt_check_gemv_kn_args(int64_t N, int64_t K, const void* x, const void* B,
                           int64_t ldb, const void* y);

/* Host-only argument check used by gemm_f16 before anything is enqueued.
 * Returns the status gemm_f16 would return for these arguments (SDT_OK when
 * the call would be launched). */
int sdt_check_gemm_args(int64_t M, int64_t N, int64_t K,
                        const void* A, int64_t lda,
                        const void* B, int64_t ldb,
                        const void* C, int64_t ldc);

/* Measurement: enqueue a register-only MFMA loop with no memory traffic in
 * the loop: `workgroups` workgroups of 8 waves (two per SIMD, the register
 * budget of the 256 x 256 GEMM kernel), each lane holding the 24 operand
 * fragments of one 64-deep k-tile of that kernel's 128 x 64 wave tile and its
 * fp32 accumulators, and performing workgroups x 8 x iters x 2^20
 * floating-point operations: with (flags & 2) == 0, iters x 64
 * v_mfma_f32_16x16x32 (the GEMM kernel's instruction and order: fragments
 * 0..7 A and 8..11 B of the first 32-deep half, 12..23 those of the second;
 * lane l holds row l % 16, elements 8 (l / 16) .. + 7 of the half); with
 * (flags & 2) != 0, iters x 32 v_mfma_f32_32x32x16 on the same fragments read
 * as four 16-deep steps (fragments 6 s .. 6 s + 3 A and 6 s + 4, 6 s + 5 B of
 * step s; lane l holds row l % 32, elements 8 (l / 32) .. + 7 of the step).
 * (flags & 1) != 0: the values are bf16 and the bf16 MFMAs run, else fp16.
 * Timed back to back on the GEMM's operand distribution it gives the matrix
 * cores' rate on that data at the part's power and clock limits, which the
 * GEMM kernel is reported against beside the nominal peak (the pages compare
 * their kernels with a power-limited ceiling measured on the part).
 * frags (device, caller-owned): 24 x 64 x 8 16-bit values, fragment f of lane
 * l at frags[(f * 64 + l) * 8 .. + 8).  out (device, caller-owned):
 * workgroups x 512 floats; thread t of workgroup w writes out[w * 512 + t],
 * the sum of its accumulator values in a fixed order.  SDT_ERR_INVALID_ARG: a
 * null pointer, iters <= 0, workgroups <= 0 or flags outside 0..3.
 * SDT_ERR_UNSUPPORTED: frags not 16-byte or out not 4-byte aligned.
 * SDT_ERR_HIP: the launch failed. */
int sdt_mfma_ceiling(const void* frags, int iters, void* out, int workgroups, int flags,
                     void* stream);

/* SDT_ABI_VERSION as the library was built. */
int sdt_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char* sdt_status_string(int status);

/* The hipError_t value recorded by the last SDT_ERR_HIP on this thread
 * (0 if none). */
int sdt_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SDT_H */
