/*
 * dense_gemm_tn.h -- C ABI of libdense_gemm_tn.so, the gfx950 TN GEMM library.
 *
 * The operation (cited by page and section):
 *   "hello-gpu, chapter 11 (GEMM-like)", section 11.1: C = A x B with
 *   C[m,n] = sum over k of A[m,k] * B[k,n]; no scaling, transpose or addend.
 *   "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", section "What we compute":
 *   the TN pairing -- A is row-major M x K, B is column-major K x N (so both
 *   operands are contiguous along K), and C is column-major.
 *
 * Storage, in elements (es = bytes per element):
 *   A[m*lda + k]   m < M, k < K    (row-major, row stride lda >= K)
 *   B[n*ldb + k]   n < N, k < K    (column n of B is K contiguous elements)
 *   C[m + n*ldc]   m < M, n < N    (column-major, ldc >= M)
 * For these TN calls, elements of A and B outside those index ranges are
 * never read, and C is written only at those M*N positions: ldc padding and
 * memory around C are left untouched (the tail rules of section 11.4 of the
 * hello-gpu chapter: out-of-range operand elements contribute zero,
 * out-of-range C is not written).  (The op-code layout calls gemm_f16 and
 * gemm_f8 relax the read rule for M- or N-contiguous operands; see there.)
 *
 * Ownership and ordering:
 *   All matrix pointers are DEVICE pointers on the current HIP device; the
 *   caller allocates and owns them.  `stream` is a hipStream_t (NULL = the
 *   default stream).  Each call validates its arguments on the host, enqueues
 *   its kernels on `stream` -- one, or two when the plan of gemm_tn_plan runs
 *   the columns of C in two parts (split-K calls add a reduction kernel) --
 *   and returns without synchronising; results are visible after the caller
 *   synchronises with the stream.  The library
 *   allocates nothing, keeps no per-call state and is safe to call from
 *   several host threads.  C must not overlap A or B.
 *
 * Errors (returned; nothing aborts):
 *   DG_ERR_INVALID_ARGUMENT  null pointer with M, N > 0; negative size;
 *                            lda or ldb < K; ldc < M; C overlapping A or B.
 *   DG_ERR_UNSUPPORTED       K, lda or ldb not a multiple of the 16-byte
 *                            vector (8 fp16 or 16 fp8 elements); A, B or C
 *                            not 16-byte aligned; one 256-row operand strip
 *                            spanning 2^31 bytes or more; more than 2^31-1
 *                            tiles in the launch.
 *   DG_ERR_HIP               the launch itself failed (hipGetLastError).
 *   M == 0 or N == 0 is a successful no-op; K == 0 writes C := 0, the empty sum.
 *   A fault inside the kernel surfaces at the caller's next synchronisation.
 */
#ifndef DENSE_GEMM_TN_H
#define DENSE_GEMM_TN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARGUMENT = 1,
  DG_ERR_UNSUPPORTED = 2,
  DG_ERR_HIP = 3
} dg_status;

/*
 * FP16 TN GEMM: A, B and C are IEEE binary16.  Products are accumulated in
 * fp32 on the matrix cores and each C element is rounded once, to nearest
 * even, from the fp32 sum.
 * Source: the FP16 GEMM of "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4",
 * section "What we compute" (TN layouts).
 */
int gemm_f16_tn(const void *A, const void *B, void *C,
                int64_t M, int64_t N, int64_t K,
                int64_t lda, int64_t ldb, int64_t ldc,
                void *stream);

/*
 * FP16 GEMM in any of the four BLAS op-code layouts, without a transpose pass.
 * C = op(A) op(B) is M x N, column-major at C[m + n*ldc] as above; op(A) is
 * M x K and op(B) is K x N:
 *   transa 'T': A[m*lda + k]  (K contiguous, lda >= K; the TN case's A)
 *   transa 'N': A[m + k*lda]  (M contiguous, lda >= M)
 *   transb 'N': B[k + n*ldb]  (K contiguous, ldb >= K; the TN case's B)
 *   transb 'T': B[k*ldb + n]  (N contiguous, ldb >= N)
 * Lower-case codes are accepted.  ('T', 'N') is exactly gemm_f16_tn, with its
 * tile configurations; the other three run 256 x 256 or 128 x 128 tiles (see
 * gemm_f16_config), each M- or N-contiguous operand staged in LDS as it lies
 * and turned by transposing LDS reads.  Rounding, ownership, ordering and the
 * C rule (only the M*N logical positions are written) are those of
 * gemm_f16_tn.  Reads differ for an M- or N-contiguous operand (A of an 'N'
 * op, B of a 'T' op): it is copied in whole K-rows of a block's 256 (or 128)
 * columns, so elements past M (or N) in a K-row -- its lda (ldb) padding or,
 * in the last block, the start of the next K-row -- may be read.  Every byte
 * read still lies inside the operand's span, [A, A + ((K-1)*lda + M)*es) for
 * A 'N' ([B, B + ((K-1)*ldb + N)*es) for B 'T'), and such elements only feed
 * outputs past M (N), which are never stored, so their values (NaN included)
 * never reach C.  K-contiguous operands keep the TN rule.  Row-major C = A B with
 * A row-major M x K and B row-major K x N (the NN indexing of section 11.1 of
 * the hello-gpu chapter) is this call with transa = transb = 'N' on the
 * operands swapped: C^T = B^T A^T, computed as gemm_f16('N', 'N', B, A, C,
 * N, M, K, ldb, lda, ldc).
 * Source: "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", section "What we
 * compute" (data in other layouts would otherwise be transposed first), and
 * "hello-gpu, chapter 11 (GEMM-like)", section 11.1.
 * Errors: DG_ERR_INVALID_ARGUMENT also for a code other than T/t/N/n and for
 * lda or ldb below the contiguous extent listed above.  DG_ERR_UNSUPPORTED
 * for lda or ldb not a multiple of 8; K not a multiple of 8 when an operand is
 * K-contiguous; M (transa 'N') or N (transb 'T') not a multiple of 8; A, B or
 * C not 16-byte aligned; one K-step of rows of an M/N-contiguous operand (64
 * K-rows) or 256 rows of a K-contiguous one spanning 2^31 bytes or more.
 */
int gemm_f16(char transa, char transb, const void *A, const void *B, void *C,
             int64_t M, int64_t N, int64_t K,
             int64_t lda, int64_t ldb, int64_t ldc,
             void *stream);

/*
 * FP8 TN GEMM: A and B are OCP FP8 E4M3FN codes (one byte each) carrying the
 * per-tensor fp32 scales scale_a and scale_b; C is bfloat16.
 *   C[m + n*ldc] = bf16_rne( fp32(scale_a * scale_b) * sum_k a(m,k) * b(k,n) )
 * with the sum accumulated in fp32 on the matrix cores.
 * Source: the FP8 GEMM of "AMD ROCm 4-wave interleave FP8 GEMM for Instinct
 * MI355X (CDNA 4)", sections "why 4 waves" and "interleave".
 */
int gemm_f8_tn(const void *A, const void *B, void *C,
               int64_t M, int64_t N, int64_t K,
               int64_t lda, int64_t ldb, int64_t ldc,
               float scale_a, float scale_b,
               void *stream);

/*
 * FP8 GEMM in any of the four BLAS op-code layouts, without a transpose pass:
 * E4M3FN A and B with per-tensor fp32 scales, bf16 C, exactly as gemm_f8_tn
 * (C = bf16_rne(fp32(scale_a * scale_b) * op(A) op(B)), fp32 accumulation),
 * with op(A), op(B) and C laid out as for gemm_f16 (elements are one byte).
 * ('T', 'N') is gemm_f8_tn.  The chunk granularity is 16 elements: lda, ldb,
 * K (when an operand is K-contiguous), M (transa 'N') and N (transb 'T') must
 * be multiples of 16, else DG_ERR_UNSUPPORTED; a K-step of an M/N-contiguous
 * operand is 128 K-rows here; other errors, and the read rule for M- or
 * N-contiguous operands, as for gemm_f16.
 * Source: the FP8 GEMM of "AMD ROCm 4-wave interleave FP8 GEMM for Instinct
 * MI355X (CDNA 4)" and, for the layouts, "FP16 GEMM optimisation on AMD RDNA 3
 * and RDNA 4", section "What we compute".
 */
int gemm_f8(char transa, char transb, const void *A, const void *B, void *C,
            int64_t M, int64_t N, int64_t K,
            int64_t lda, int64_t ldb, int64_t ldc,
            float scale_a, float scale_b,
            void *stream);

/*
 * Strided-batched Q K^T (fp16 in, fp16 out, fp32 accumulate): for each head
 * h < batch,
 *   S[h*stride_s + j*lds + i] = sum_d Q[h*stride_q + i*ldq + d] * Kmat[h*stride_k + j*ldk + d]
 * for i < M (query rows), j < N (key rows), d < D (head dim).  Q_h is the
 * row-major A and K_h, row-major N x D, is exactly the K-contiguous B of the TN
 * product, so S_h is column-major with leading dimension lds (>= M): seen as a
 * row-major [N][lds] array it holds S_h transposed.  Swapping Q and Kmat (and
 * M and N) gives the row-major S_h.
 * Source: the QK^T kernel sketch of the mlqm.cn TileLang attention page
 * (K dimension = head dim 128).  Strides are in elements; ldq, ldk >= D,
 * lds >= M; the per-head regions of S must not overlap (stride_s >= lds*N
 * when batch > 1), otherwise DG_ERR_INVALID_ARGUMENT.  ldq, ldk, stride_q and
 * stride_k must be multiples of 8 (16-byte rows and heads of Q and K), else
 * DG_ERR_UNSUPPORTED; lds and stride_s may be any value: S is stored 16 bytes
 * at a time when both are multiples of 8, 8 bytes at a time when both are
 * multiples of 4, element by element otherwise.
 */
int gemm_batched_qkt(const void *Q, const void *Kmat, void *S,
                     int64_t batch, int64_t M, int64_t N, int64_t D,
                     int64_t ldq, int64_t ldk, int64_t lds,
                     int64_t stride_q, int64_t stride_k, int64_t stride_s,
                     void *stream);

/*
 * Fused softmax attention forward (fp16 in, fp16 out; fp32 scores, fp32
 * accumulation, probabilities rounded to fp16 for the second product): for
 * each head h < batch and query row i < M,
 *   s_n     = scale * sum_d Q[h*stride_q + i*ldq + d] * K[h*stride_k + n*ldk + d]
 *   O[h*stride_o + i*ldo + d] = sum_n exp(s_n - max s) * Vt[h*stride_v + d*ldv + n]
 *                               / sum_n exp(s_n - max s)
 * over keys n < N, for d < D.  The score matrix is never written to memory.
 * Source: the chapter summary of "hello-gpu, chapter 11 (GEMM-like)" (the
 * next step after the GEMM joins it with softmax so the intermediate result
 * need not go back to memory) and the fused attention of the mlqm.cn TileLang
 * attention page; the pages give no formula, so the operation is the textbook
 * softmax attention.  Both products are TN products (each operand contiguous
 * along the summed dimension), which is why V is passed transposed: Vt is
 * D rows of N keys (row d = column d of V), e.g. the column-major output of
 * the V projection computed with gemm_f16_tn.
 *
 * Sizes and storage (strides in elements): Q row-major M x D (ldq >= D), K
 * row-major N x D (ldk >= D), Vt row-major D x N (ldv >= N), O row-major
 * M x D (ldo >= D).  D must be 128 (else DG_ERR_UNSUPPORTED).  Pointers must
 * be 16-byte aligned and all ld and stride values multiples of 8 (else
 * DG_ERR_UNSUPPORTED).  Input head strides may be 0 (one K/V shared by all
 * heads); the heads of O must not overlap (stride_o >= (M-1)*ldo + D when
 * batch > 1) and O must not overlap Q, K or Vt (else DG_ERR_INVALID_ARGUMENT).
 * scale must be finite and >= 0; N must be >= 1 when M > 0 (softmax over no
 * keys is undefined); negative sizes or strides and null pointers are
 * DG_ERR_INVALID_ARGUMENT.  batch == 0 or M == 0 is a successful no-op.
 * Per-head extents of Q, K (plus 64 rows) and Vt (plus 64 keys) must stay
 * below 2^31 bytes (else DG_ERR_UNSUPPORTED).  Elements of Q, K and Vt
 * outside their logical extents (ld padding, head gaps) are never read, and
 * O is written only at its batch x M x D logical positions.  Device pointers, stream and ordering as
 * for the GEMM entry points above; one kernel launch, no allocation.
 */
int attention_fwd_f16(const void *Q, const void *K, const void *Vt, void *O,
                      int64_t batch, int64_t M, int64_t N, int64_t D,
                      int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo,
                      int64_t stride_q, int64_t stride_k, int64_t stride_v, int64_t stride_o,
                      float scale, void *stream);

/* Static, NUL-terminated name of a dg_status value ("unknown status" otherwise). */
const char *gemm_status_string(int status);

/*
 * Host-side view of the block -> tile order used by every kernel above (the
 * grouped order of "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", Step 6,
 * composed with the chiplet-aware remap of the MI355X FP8 GEMM page).  For a
 * launch over `batch` heads of tiles_m x tiles_n tiles, writes for every
 * hardware block id b the triple (head, tile_m, tile_n) to out[3*b .. 3*b+2].
 * `out` is a HOST buffer of 3*batch*tiles_m*tiles_n int64 values.  Returns
 * DG_ERR_INVALID_ARGUMENT for a null `out` or non-positive sizes.
 * For measurement only, the environment variable DG_TILE_ORDER = grouped
 * (the grouped order without the chiplet remap) or row (consecutive blocks
 * along a row of tiles) changes the order the TN calls (gemm_f16_tn,
 * gemm_f8_tn, gemm_batched_qkt) use; this function always reports the
 * library's own order.
 */
int gemm_tile_order(int64_t tiles_m, int64_t tiles_n, int64_t batch, int64_t *out);

/* Output tile edge (rows of C per block) of the main, 256-row kernel. */
int gemm_block_tile(void);

/*
 * The kernel configuration of a single launch of the GEMM entry points for a
 * problem of the given sizes on the current HIP device (fp8 != 0: one-byte
 * elements, else fp16; gemm_tn_plan tells when a TN call splits its columns
 * over two launches instead).  One tile shape does not suit every size, so the library has a small
 * set and a selector ("FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4",
 * sections "Final results" and "Further tuning"):
 *   0  256 x 256 output tiles, one block per CU, pipelined K loop;
 *   1  256 x 224 tiles (fewer rounds of one block per CU for some widths);
 *   2  128 x 128 tiles, two blocks per CU (grids the wide tiles leave idle);
 *   3  the skinny-K kernel (K * element bytes <= 256);
 *   4  256 x 256 tiles computed by 8 waves in two groups that alternate
 *      between reading fragments and multiplying ("ping-pong"; the design the
 *      "AMD ROCm 4-wave interleave FP8 GEMM for Instinct MI355X (CDNA 4)" page
 *      weighs against its 4-wave one); only chosen when forced;
 *  -1  negative sizes.
 * The choice is a pure function of the sizes and the device's CU count.  For
 * measurement and tests, the environment variable DG_GEMM_TILE = 256, 224,
 * 128 or pingpong forces configuration 0, 1, 2 or 4 for every non-skinny
 * problem.
 */
int gemm_tn_config(int fp8, int64_t M, int64_t N, int64_t K, int64_t batch);

/*
 * LDS stages of the K ring the 128 x 128 kernel (configuration 2 in every
 * layout, and the partial-product kernel of the split-K calls) uses for a grid
 * of `blocks` blocks of `ksteps` K-steps each (64 fp16 or 128 fp8 elements per
 * step) on the current HIP device: 4 (a 128 KiB ring, copies three steps ahead, one
 * block per compute unit) when the grid has at most one block per compute
 * unit and ksteps >= 8 -- there no second block covers a step whose copies
 * wait on DRAM -- else 2 (64 KiB, two blocks per compute unit).  The number
 * of LDS buffers is traded against occupancy and chosen by measurement per
 * shape ("FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", step 8 and
 * section "Further tuning").  -1 for negative arguments.  A query for
 * measurement labels and tests; results are identical either way.
 */
int gemm_mid_stages(int64_t blocks, int64_t ksteps);

/*
 * Kernel configuration gemm_f16 picks for op codes (transa, transb) and an
 * M x N x K problem: for ('T', 'N') that of gemm_tn_config; for the other
 * layouts 0 (256 x 256) or 2 (128 x 128) -- the 224-wide and skinny-K
 * kernels take K-contiguous operands only, and the selector's choice between
 * the remaining two is the same cost comparison.  Returns -1 for an invalid
 * code or a negative size.  DG_GEMM_TILE = 256 or 224 forces configuration 0
 * and 128 configuration 2 for the other layouts (K > 128).
 */
int gemm_f16_config(char transa, char transb, int64_t M, int64_t N, int64_t K);

/* The same for gemm_f8 (TN: gemm_tn_config with fp8 != 0). */
int gemm_f8_config(char transa, char transb, int64_t M, int64_t N, int64_t K);

/*
 * Split-K TN GEMM for grids of few output tiles with a long K (small M x N,
 * large K), where one block per tile would leave most compute units idle.
 * Same product, rounding, validation and ownership as gemm_f16_tn /
 * gemm_f8_tn; in addition K is cut into at most `splits` ranges of whole
 * K-steps (64 fp16 or 128 fp8 elements), each multiplied into an fp32 partial
 * in the caller's `workspace`, and a second kernel on the same stream sums
 * the partials in range order (deterministic) and rounds once into C.  The
 * result differs from the unsplit call only by fp32 summation order.
 *   splits     1 .. 64; 1 (or a K too short to split) is exactly gemm_*_tn
 *              and does not touch the workspace.  gemm_splitk_choose suggests
 *              a count.
 *   workspace  device memory, 16-byte aligned, at least
 *              gemm_splitk_workspace_bytes(M, N, splits) bytes, overlapping
 *              none of A, B and C; owned by the caller, contents undefined
 *              afterwards, and it must not be used by other work on another
 *              stream until this call's kernels have run.
 * Errors: as for gemm_f16_tn / gemm_f8_tn, plus DG_ERR_INVALID_ARGUMENT for
 * splits outside 1 .. 64, a null or too-small workspace (when the call does
 * split) or one overlapping an operand, and DG_ERR_UNSUPPORTED for a
 * misaligned one.
 * Source: "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", sections "Final
 * results" and "Further tuning" (one tile configuration is wrong for small or
 * skinny products; a library needs a set of configurations and a selector).
 */
int gemm_f16_tn_splitk(const void *A, const void *B, void *C,
                       int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldb, int64_t ldc,
                       int64_t splits, void *workspace, int64_t workspace_bytes,
                       void *stream);
int gemm_f8_tn_splitk(const void *A, const void *B, void *C,
                      int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldc,
                      float scale_a, float scale_b,
                      int64_t splits, void *workspace, int64_t workspace_bytes,
                      void *stream);

/*
 * Plans for grids with a ragged last round.  The 256-row kernel runs one block
 * per compute unit, so a grid of T tiles takes ceil(T / CUs) rounds however
 * few tiles the last round holds (4096 x 4608 in 256 x 256 tiles: 288 tiles,
 * a second round of 32 on 256 CUs).  The TN calls (gemm_f16_tn, gemm_f8_tn,
 * gemm_batched_qkt for K * es > 256, and the *_ws calls below) then may run the
 * first dp_cols columns of C as whole rounds of the 256-row kernel and the
 * remaining columns as a second launch on the same stream, in the
 * configuration gemm_tn_config gives for that narrower product.  Every
 * element is then computed exactly as by a single launch (the same products
 * in the same K order): only the time changes.  With a caller workspace (the
 * *_ws calls) the remaining columns may instead have their K range cut into
 * `splits` ranges summed through the workspace (as gemm_f16_tn_splitk), which
 * spreads the few tail tiles over every compute unit -- the data-parallel
 * plus split-tail schedule that stream-K generalises -- and a product of few
 * tiles with a long K may be split-K as a whole; such plans differ from the
 * single launch by the fp32 summation order only.  Plans are chosen with a
 * time model fitted to MI355X measurements and taken only when modelled at
 * least 5 % faster than the single launch; DG_GEMM_TILE (see gemm_tn_config)
 * turns them off.
 * Source: "FP16 GEMM optimisation on AMD RDNA 3 and RDNA 4", section "Further
 * tuning" (per-shape configurations and their selection).
 *
 * gemm_f16_tn_ws / gemm_f8_tn_ws: gemm_f16_tn / gemm_f8_tn by the plan that
 *   fits `workspace_bytes` bytes of `workspace` (device memory; NULL with 0
 *   bytes allowed: then only plans without a workspace).  The bytes a plan
 *   uses, the first gemm_tn_plan(...)[4] of the workspace, must be 16-byte
 *   aligned and overlap none of A, B and C.  Ownership, ordering and the C
 *   rule are those of gemm_f16_tn; the workspace is the caller's, the bytes
 *   used are undefined afterwards (the rest is not touched), and calls that
 *   may run concurrently must not share it.  Errors: as gemm_f16_tn, plus
 *   DG_ERR_INVALID_ARGUMENT for negative workspace_bytes, a NULL workspace
 *   with nonzero bytes, or used bytes overlapping A, B or C, and
 *   DG_ERR_UNSUPPORTED for a misaligned workspace whose plan uses it.
 * gemm_tn_workspace_bytes: bytes of workspace the best plan for an M x N x K
 *   product uses (0 when it needs none; -1 for negative sizes).
 * gemm_tn_plan: the plan for the given sizes, head count and workspace bytes:
 *   out[0] the single launch's configuration (as gemm_tn_config), out[1]
 *   dp_cols (0: the columns are not split), out[2] the configuration of the
 *   dp_cols columns (0 or 1; -1 when not split), out[3] the K ranges of the
 *   remaining columns (of the whole product when out[1] is 0; 1: not split),
 *   out[4] the workspace bytes used.  DG_ERR_INVALID_ARGUMENT for a NULL out
 *   or negative arguments.
 */
int gemm_f16_tn_ws(const void *A, const void *B, void *C,
                   int64_t M, int64_t N, int64_t K,
                   int64_t lda, int64_t ldb, int64_t ldc,
                   void *workspace, int64_t workspace_bytes, void *stream);
int gemm_f8_tn_ws(const void *A, const void *B, void *C,
                  int64_t M, int64_t N, int64_t K,
                  int64_t lda, int64_t ldb, int64_t ldc,
                  float scale_a, float scale_b,
                  void *workspace, int64_t workspace_bytes, void *stream);
int64_t gemm_tn_workspace_bytes(int fp8, int64_t M, int64_t N, int64_t K);
int gemm_tn_plan(int fp8, int64_t M, int64_t N, int64_t K, int64_t batch,
                 int64_t workspace_bytes, int64_t *out);

/*
 * Per-block clock records, a measurement facility (off by default).  After
 * gemm_clock_record(buf, records) with a device buffer of `records` records
 * of ten uint64 words (80 bytes each, 8-byte aligned), every launch of the
 * calls above takes one record per block, in launch order, while they fit
 * (a launch that does not fit whole records nothing; the split-K reduction
 * kernel records nothing).  Words 2p and 2p+1 of a block's record hold the
 * shader-clock counter and the constant 100 MHz counter at point p: 0 the
 * block's start, 1 the start of its pipelined K loop, 2 the end of that loop,
 * 3 after its first wave's last stores completed (points 1 and 2 are left
 * zero by kernels without a pipelined K loop: the 128 x 128, skinny-K,
 * ping-pong and attention kernels); word 8 is the XCD it ran on and word 9
 * its block index.  Counter ticks over real-time ticks are the clock it ran at.
 * gemm_clock_record(NULL, 0) turns recording off; gemm_clock_records_used()
 * returns the records taken (or asked for, if more) since the last
 * gemm_clock_record call.  The setting is process-wide; the buffer must stay
 * valid while recording is on.  Errors: DG_ERR_INVALID_ARGUMENT for a
 * negative count or a NULL buffer with a nonzero count (or the reverse),
 * DG_ERR_UNSUPPORTED for a misaligned buffer.
 * Source: the benchmarking method of "AMD ROCm 4-wave interleave FP8 GEMM for
 * Instinct MI355X (CDNA 4)", section "Hardware platform and chiplet-aware
 * optimisation" (per-XCD behaviour of the 8-chiplet part), and the RDNA page's
 * section "Measuring resources" (timing what the kernel does).
 */
int gemm_clock_record(void *buf, int64_t records);
int64_t gemm_clock_records_used(void);

/*
 * gemm_f16_tn_splitk without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the fp32 partials live in a static
 * 32 MiB device array of the library (one per device, held until the process
 * ends), so the call itself allocates nothing.  Same product, validation and
 * result as gemm_f16_tn_splitk with the same `splits` (bit for bit), plus:
 *   DG_ERR_UNSUPPORTED  splits * N * (M rounded up to 4) * 4 bytes > 32 MiB
 *                       (gemm_splitk_workspace_bytes(M, N, splits) > 2^25);
 *   DG_ERR_HIP          the array's device address could not be looked up.
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device (e.g. on two streams without ordering) race; calls
 * ordered on one stream do not.
 */
int gemm_f16_tn_splitk_noalloc(const void *A, const void *B, void *C,
                               int64_t M, int64_t N, int64_t K,
                               int64_t lda, int64_t ldb, int64_t ldc,
                               int64_t splits, void *stream);

/* Workspace bytes the split-K calls need for M x N and `splits`:
 * splits * N * (M rounded up to 4) * 4; -1 for invalid arguments. */
int64_t gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t splits);

/* Suggested split count for an M x N x K TN product (fp8 != 0: FP8): as many
 * splits of the 128 x 128 tiles as fit one block per compute unit, doubled to
 * two per compute unit when those one-per-unit ranges are 64 K-steps or longer
 * (the doubled ranges then keep at least 32), each keeping at least 16 K-steps
 * and at most 64 splits.  Between half and all of the compute units' worth of
 * tiles: the count that fits two blocks per unit in one round, when the
 * busiest unit's block-steps drop to at most 0.8 of the unsplit K-steps, else
 * 1.  1 for a grid of at least one tile per compute unit.  -1 for negative
 * sizes. */
int64_t gemm_splitk_choose(int fp8, int64_t M, int64_t N, int64_t K);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_TN_H */
