/*
 * gemm_f32.h -- C ABI of libgemm_f32.so: row-major FP32 matrix
 * multiplication C = A x B on an AMD MI355X (gfx950).
 *
 * Operation (every compute entry point):
 *
 *   C[i * ldc + j] = sum over k < K of A[i * lda + k] * B[k * ldb + j]
 *                    for 0 <= i < M, 0 <= j < N.
 *
 *   Each output cell is the dot product of row i of A and column j of B
 *   ("Tiled Matrix Multiplication in CUDA", section 1; "Tiled GEMM: Matrix
 *   Multiplication in CUDA", section 1).  Matrices are row-major, cell (r, c)
 *   at flat index r * ld + c ("Tiled Matrix Multiplication in CUDA",
 *   section 2); A is M x K, B is K x N and C is M x N ("Tiled GEMM: Matrix
 *   Multiplication in CUDA", section 7.1, rectangular shapes).  The leading
 *   dimensions lda, ldb, ldc let each operand be a row-major sub-matrix of a
 *   wider allocation.
 *
 * Arithmetic: FP32 multiplies and FP32 accumulation (round to nearest even).
 * No reduced-precision input formats are used.  The summation order depends
 * on the kernel, so float results of different kernels agree within
 * rounding; each kernel is deterministic run to run.  Integer-valued inputs
 * whose partial sums stay below 2^24 in magnitude give exact results.
 *
 * Memory and ownership: A, B and C are device pointers (or any pointer the
 * GPU can dereference), 4-byte aligned, owned by the caller.  The library
 * allocates nothing on these calls and keeps no pointer after returning.
 * C is overwritten in its M x N region only; the padding columns
 * ldc - N of every row, and everything outside the region, are never read
 * or written.  C must not overlap A or B.  A and B are read only inside
 * their storage, from the first element to the last element of the last
 * row; the kernels may read padding elements between rows, whose values
 * (NaN included) never reach C.
 *
 * Streams and threading: every compute call only enqueues work on `stream`
 * (a hipStream_t; NULL means the null stream) and returns; the caller
 * synchronises.  Calls are reentrant.
 *
 * Errors: arguments are validated before anything is enqueued; on a
 * negative return nothing was enqueued, except for GEMM_F32_EHIP, which
 * reports a failed launch.  The library never aborts.  gemm_f32_last_error()
 * describes the most recent failure on the calling thread.
 */
#ifndef GEMM_F32_H
#define GEMM_F32_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define GEMM_F32_OK 0
#define GEMM_F32_EINVAL (-1)    /* invalid sizes, leading dims, pointers */
#define GEMM_F32_EHIP (-2)      /* a HIP runtime call or launch failed */
#define GEMM_F32_ENOKERNEL (-3) /* no such variant or tile configuration */

/* Operand forms for gemm_f32_ex. */
#define GEMM_F32_OP_N 0 /* as stored */
#define GEMM_F32_OP_T 1 /* transposed */

/* Kernel variants, in the order the pages build them up. */
#define GEMM_F32_VARIANT_NAIVE 0    /* one thread per output cell */
#define GEMM_F32_VARIANT_LDS 1      /* LDS (shared-memory) tiles, 2 barriers */
#define GEMM_F32_VARIANT_REGBLOCK 2 /* per-thread register patch, VALU FMA */
#define GEMM_F32_VARIANT_MFMA 3     /* FP32 matrix cores, double-buffered */
#define GEMM_F32_NUM_VARIANTS 4

/*
 * gemm_f32 -- C = A x B with the kernel and tile configuration the library
 * selects for the shape ("Tiling and Blocking for Reuse", "choosing the tile
 * size"): a built-in table of shapes tuned by measurement on MI355X, and for
 * other shapes a cost model whose per-CU rates were measured there (it
 * accounts for how many tiles each CU receives and runs at once).  The model
 * may split C in two parts with different tile sizes, run as two launches
 * on `stream` (gemm_f32_plan reports how).
 *
 *   M, N, K    sizes, 0 <= M, N, K <= 2^31 - 1
 *   A, lda     M x K operand, lda >= max(1, K)
 *   B, ldb     K x N operand, ldb >= max(1, N)
 *   C, ldc     M x N result, ldc >= max(1, N)
 *   stream     hipStream_t to enqueue on, or NULL
 *
 * M == 0 or N == 0: returns GEMM_F32_OK and enqueues nothing.
 * K == 0: C's M x N region is set to zero (the empty sum).
 * A pointer may be NULL only when its matrix has no elements.
 * Returns GEMM_F32_OK, GEMM_F32_EINVAL or GEMM_F32_EHIP.
 */
int gemm_f32(int64_t M, int64_t N, int64_t K,
             const float *A, int64_t lda,
             const float *B, int64_t ldb,
             float *C, int64_t ldc,
             void *stream);

/*
 * gemm_f32_variant -- the same operation with an explicit kernel.
 *
 *   variant    one of GEMM_F32_VARIANT_*
 *   config_id  index of a compiled tile configuration of that variant
 *              (0 <= config_id < gemm_f32_config_count(variant)), or -1 for
 *              the configuration the library would pick for this shape as
 *              one launch (never split as gemm_f32 may split it)
 *
 * The naive kernel follows "Tiled Matrix Multiplication in CUDA", section 5
 * (with the bounds guard of "Tiling and Blocking for Reuse"); the LDS kernel
 * follows the phase loop of "Tiled GEMM: Matrix Multiplication in CUDA",
 * sections 2 and 4, with the zero-filled loads of its section 7.1; the
 * register-blocked kernel follows "Tiling and Blocking for Reuse", "the next
 * level: register blocking"; the MFMA kernel adds the double buffering of
 * "Tiled GEMM: Matrix Multiplication in CUDA", section 8.
 *
 * Other arguments and all semantics are those of gemm_f32.  Returns
 * GEMM_F32_ENOKERNEL for an unknown variant or configuration.
 */
int gemm_f32_variant(int variant, int config_id,
                     int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     float *C, int64_t ldc,
                     void *stream);

/*
 * gemm_f32_strided_batched -- `batch` independent products
 *
 *   C_b = A_b x B_b,  X_b = X + b * strideX (in floats),  0 <= b < batch,
 *
 * each with the semantics of gemm_f32 (same M, N, K and leading dimensions
 * for every product).  The products are the independent output tiles of the
 * pages' decomposition ("Tiled Matrix Multiplication in CUDA", section 1:
 * every cell of C is independent) laid out over one more index; the pages
 * motivate GEMM by attention and mixture-of-experts layers, which are
 * batches of such products.
 *
 *   batch          0 <= batch <= 2^31 - 1; 0 enqueues nothing
 *   strideA/B      >= 0; 0 reuses one A (or B) for every product
 *   strideC        >= (M - 1) * ldc + N when batch > 1, so the products'
 *                  C regions do not overlap; batch * stride must stay below
 *                  2^58 floats
 *
 * No C region may overlap any A or B region (checked on the address ranges
 * spanned by the whole batch).  The configuration is chosen from the shape
 * of one product and the total number of tiles; every product may be split
 * in two parts as gemm_f32 splits one (two launches over the whole batch).
 * Returns as gemm_f32.
 */
int gemm_f32_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                             const float *A, int64_t lda, int64_t strideA,
                             const float *B, int64_t ldb, int64_t strideB,
                             float *C, int64_t ldc, int64_t strideC,
                             void *stream);

/* gemm_f32_strided_batched with an explicit kernel, as gemm_f32_variant. */
int gemm_f32_strided_batched_variant(int variant, int config_id,
                                     int64_t batch, int64_t M, int64_t N, int64_t K,
                                     const float *A, int64_t lda, int64_t strideA,
                                     const float *B, int64_t ldb, int64_t strideB,
                                     float *C, int64_t ldc, int64_t strideC,
                                     void *stream);

/*
 * gemm_f32_ex -- the general form: transposed operands, a batch, and an
 * optional explicit kernel.
 *
 *   C_b = op(A_b) x op(B_b),  0 <= b < batch,
 *
 *   op(A) = A (opA = GEMM_F32_OP_N; A stored M x K, lda >= max(1, K)) or A^T
 *           (GEMM_F32_OP_T; A stored K x M row-major, lda >= max(1, M), so
 *           op(A)[i][k] = A[k * lda + i]);
 *   op(B) = B (opB = GEMM_F32_OP_N; B stored K x N, ldb >= max(1, N)) or B^T
 *           (GEMM_F32_OP_T; B stored N x K, ldb >= max(1, K), so
 *           op(B)[k][j] = B[j * ldb + k]).
 *
 * Row-major flat indexing is the pages' layout ("Tiled Matrix
 * Multiplication in CUDA", section 2); the page names column-major storage
 * as the other order, and a column-major M x K matrix with leading
 * dimension ld is exactly the row-major K x M matrix that GEMM_F32_OP_T
 * describes.  Column-major C = A x B can also be had without transposes as
 * the row-major product C^T = B^T x A^T, i.e. gemm_f32 with the operands
 * swapped.
 *
 *   variant, config_id   -1, -1 for the library's choice, else as in
 *                        gemm_f32_variant.  Transposed operands are taken by
 *                        the naive kernel and by the MFMA configurations
 *                        that list them; others return GEMM_F32_ENOKERNEL.
 *   batch, strides       as in gemm_f32_strided_batched (batch 1, strides 0
 *                        for one product).
 *
 * Returns as gemm_f32; GEMM_F32_EINVAL for an unknown opA or opB.
 */
int gemm_f32_ex(int variant, int config_id, int opA, int opB,
                int64_t batch, int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda, int64_t strideA,
                const float *B, int64_t ldb, int64_t strideB,
                float *C, int64_t ldc, int64_t strideC,
                void *stream);

/*
 * gemm_f32_splitk -- C = A x B computed as `splits` partial products over
 * slices of K, for shapes with too few output tiles to fill the GPU (small
 * or ragged products; "Tiling and Blocking for Reuse", "choosing the tile
 * size": tail effects and occupancy bound the tile choice).
 *
 *   C = sum over s of A[:, K_s] x B[K_s, :],  K_s = [s * L, min((s + 1) L, K))
 *
 * L is ceil(K / splits) rounded up to a multiple of 32; the number of
 * slices actually used is ceil(K / L) <= splits.  Each partial product
 * goes to its own M x N slice of `workspace` (packed rows), then one more
 * kernel adds the slices into C in ascending s for every element, so the
 * result is deterministic.
 *
 *   variant, config_id  kernel of the partial products, as in gemm_f32_ex
 *                       (-1, -1: the library's choice)
 *   splits              1 .. 65535, or 0 for the library's choice (enough
 *                       128 x 128 tiles to give every CU of the GPU one, at
 *                       least 1024 k per split); one slice is the plain
 *                       product and needs no workspace
 *   workspace           device memory of at least
 *                       gemm_f32_splitk_workspace_size(M, N, K, splits)
 *                       bytes, 4-byte aligned, owned by the caller, not
 *                       overlapping A, B or C; its contents are overwritten
 *   others              as in gemm_f32
 *
 * Returns as gemm_f32 (GEMM_F32_EINVAL also for a missing or short
 * workspace).
 */
int gemm_f32_splitk(int variant, int config_id, int64_t splits,
                    int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda,
                    const float *B, int64_t ldb,
                    float *C, int64_t ldc,
                    void *workspace, int64_t workspace_bytes,
                    void *stream);

/*
 * gemm_f32_splitk_noalloc -- gemm_f32_splitk for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc): the partial products go to a scratch
 * array the library holds in device memory instead of a workspace argument.
 *
 * The scratch is a static device array of GEMM_F32_SPLITK_SCRATCH_BYTES
 * bytes; every GPU the library runs on holds its own copy until the process
 * ends.  Its device address is looked up on the first call on each device
 * (hipGetSymbolAddress, with that device current); the call itself performs
 * no allocation and no hipMalloc / hipFree.  Every call on one GPU uses that
 * GPU's one array, so calls that overlap in time on the same GPU (other
 * streams, other threads) race and must be serialised by the caller.
 *
 * Arguments and results are those of gemm_f32_splitk without the
 * workspace; splits = 0 takes the library's choice capped at the number of
 * M x N slices that fit the scratch (at most one slice: the plain product).
 * Returns GEMM_F32_EINVAL when the partial products need more
 * than GEMM_F32_SPLITK_SCRATCH_BYTES (gemm_f32_splitk_workspace_size tells
 * how much they need), and GEMM_F32_EHIP when the scratch address cannot be
 * obtained.
 */
#define GEMM_F32_SPLITK_SCRATCH_BYTES 33554432 /* 32 MiB */
int gemm_f32_splitk_noalloc(int variant, int config_id, int64_t splits,
                            int64_t M, int64_t N, int64_t K,
                            const float *A, int64_t lda,
                            const float *B, int64_t ldb,
                            float *C, int64_t ldc,
                            void *stream);

/* Bytes of workspace gemm_f32_splitk needs for these arguments, splits = 0
   meaning the library's choice (0 when it needs none, or for invalid
   sizes). */
int64_t gemm_f32_splitk_workspace_size(int64_t M, int64_t N, int64_t K, int64_t splits);

/* Static description of a return code; never NULL. */
const char *gemm_f32_strerror(int code);

/*
 * Detail of the most recent failing call on the calling thread (for example
 * which argument was invalid); an empty string if none failed.  The pointer
 * stays valid until the next library call on the same thread.
 */
const char *gemm_f32_last_error(void);

/* Number of compiled tile configurations of a variant, or GEMM_F32_ENOKERNEL. */
int gemm_f32_config_count(int variant);

/*
 * Name of a tile configuration, e.g. "mfma2d_256x256x32_w4x4_swz_g4_il";
 * NULL when the variant or configuration does not exist.  Static storage.
 */
const char *gemm_f32_config_name(int variant, int config_id);

/*
 * The variant and configuration gemm_f32 would run for these arguments
 * (sizes and leading dimensions only; no pointer is dereferenced).  Where
 * gemm_f32 splits the product in two launches (see gemm_f32_plan), the
 * configuration of the first.  Returns GEMM_F32_OK or GEMM_F32_EINVAL.
 */
int gemm_f32_select(int64_t M, int64_t N, int64_t K,
                    int64_t lda, int64_t ldb, int64_t ldc,
                    int *variant, int *config_id);

/*
 * How gemm_f32 runs one product with these sizes and leading dimensions:
 * *parts = 1 (one launch of variant[0], config_id[0]) or 2.  With 2, C is
 * split along *axis (0: rows, 1: columns) after *split rows (columns): the
 * first part runs variant[0], config_id[0] and the rest variant[1],
 * config_id[1], one launch each, in that order, on the same stream.  The
 * split exists because the last wave of large output tiles can be mostly
 * empty ("Tiling and Blocking for Reuse", choosing the tile size: tail
 * effects); the first part takes large tiles in whole waves across all CUs
 * and the rest the cost model's choice for what remains, when the model
 * predicts at least 2% less time.  variant and config_id point to arrays of
 * two; with one part both entries describe it.  Returns GEMM_F32_OK or
 * GEMM_F32_EINVAL.
 */
int gemm_f32_plan(int64_t M, int64_t N, int64_t K,
                  int64_t lda, int64_t ldb, int64_t ldc,
                  int *parts, int *axis, int64_t *split, int *variant, int *config_id);

/* ABI version of this header: 3 (2 added gemm_f32_plan, 3
   gemm_f32_splitk_noalloc). */
int gemm_f32_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F32_H */
