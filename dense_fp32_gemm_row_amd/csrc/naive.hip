// Stage 1: one thread per output cell, the whole dot product read from
// global memory.
//
// Prior art: the naive kernel of "Tiled Matrix Multiplication in CUDA",
// section 5, with the bounds guard of "Tiling and Blocking for Reuse" ("why
// naive is slow").  Each thread walks row i of A (k moves along the row) and
// column j of B (k moves down the column) and adds the products into one
// FP32 register in ascending k with fused multiply-adds.
//
// gfx950 mapping.  A workgroup is BX x BY threads; threadIdx.x runs along the
// columns of C and threadIdx.y along the rows, every row index built from .y
// parts only and every column index from .x parts only (the axis rule of
// section 4 of the same page).  With BX = 64 one wavefront covers 64
// consecutive columns of one row, so its reads of B and its store of C are
// 256-byte contiguous and its read of A is one broadcast address.
//
// Transposed operands only change the two element strides of each operand.
//
// Roofline: 2 FLOP per 8 requested bytes (0.25 FLOP/B, "Tiled GEMM: Matrix
// Multiplication in CUDA", section 1) -- HBM bound on paper; caches serve
// most of the re-reads in practice.

#include "gemm_internal.h"

namespace gemm_f32_impl {
namespace {

// Element (i, k) of op(A) sits at A[i * a_ri + k * a_rk] and element (k, j)
// of op(B) at B[k * b_rk + j * b_rj]: (lda, 1) and (ldb, 1) for operands
// as stored, (1, lda) and (1, ldb) for transposed ones.
template <int BX, int BY>
__global__ __launch_bounds__(BX * BY) void gemm_naive_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t a_ri, int64_t a_rk,
    const float *__restrict__ B, int64_t b_rk, int64_t b_rj, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n, BatchArgs bt) {
    const int tile = batch_select(blockIdx.x, tiles_m * tiles_n, bt, A, B, C, K);
    const int tile_row = tile / tiles_n;
    const int tile_col = tile - tile_row * tiles_n;
    const int row = tile_row * BY + threadIdx.y;  // vertical parts only
    const int col = tile_col * BX + threadIdx.x;  // horizontal parts only
    if (row >= M || col >= N) return;

    const float *a = A + static_cast<int64_t>(row) * a_ri;
    const float *b = B + static_cast<int64_t>(col) * b_rj;
    float acc = 0.0f;
    for (int k = 0; k < K; ++k) {
        acc = fmaf(*a, *b, acc);
        a += a_rk;
        b += b_rk;
    }
    C[static_cast<int64_t>(row) * ldc + col] = acc;
}

template <int BX, int BY>
hipError_t launch_naive(const Problem &p, hipStream_t stream) {
    const int tiles_n = ceil_div(p.N, BX);
    const int tiles_m = ceil_div(p.M, BY);
    const int64_t grid = static_cast<int64_t>(tiles_n) * tiles_m * p.batch;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_naive_kernel<BX, BY>), dim3(static_cast<unsigned>(grid)),
                       dim3(BX, BY), 0, stream, p.M, p.N, p.K, p.A,
                       p.ta ? int64_t{1} : p.lda, p.ta ? p.lda : int64_t{1}, p.B,
                       p.tb ? int64_t{1} : p.ldb, p.tb ? p.ldb : int64_t{1}, p.C, p.ldc, tiles_m,
                       tiles_n, batch_of(p));
    return hipGetLastError();
}

const ConfigEntry kNaiveConfigs[] = {
    {"naive_64x4", launch_naive<64, 4>, kCapTransposed},
    {"naive_16x16", launch_naive<16, 16>, kCapTransposed},
    {"naive_64x1", launch_naive<64, 1>, kCapTransposed},
};

}  // namespace

const ConfigEntry *naive_configs(int *count) {
    *count = static_cast<int>(sizeof(kNaiveConfigs) / sizeof(kNaiveConfigs[0]));
    return kNaiveConfigs;
}

}  // namespace gemm_f32_impl
