// Stage 2: shared-memory (LDS) tiling in phases.
//
// Prior art: the tiled kernels of "Tiled Matrix Multiplication in CUDA",
// section 7, and "Tiled GEMM: Matrix Multiplication in CUDA", sections 2
// and 4.  A T x T workgroup computes one T x T tile of C.  The K dimension is
// walked in phases of T: every thread copies one element of the current A
// tile and one of the current B tile into LDS, the workgroup waits (the
// read-after-write barrier), every thread adds T products from LDS into its
// register, and the workgroup waits again before the tiles are overwritten
// (the write-after-read barrier).  Each element fetched from global memory is
// reused T times, so requested traffic falls by T and the arithmetic
// intensity rises to T / 4 FLOP per byte ("Tiled GEMM: Matrix Multiplication
// in CUDA", section 2, the intensity table).
//
// Ragged shapes ("Tiled GEMM: Matrix Multiplication in CUDA", section 7.1):
// the grid is rounded up, loads outside A or B write 0.0 into LDS so the
// extra products add nothing, and the store is guarded.
//
// Padding (section 7.2 of the same page): the row reads of tileA are
// broadcasts and the column reads of tileB hit consecutive banks, so this
// kernel needs no padding; the PAD = 1 configurations exist to show that in
// the bank-conflict counters.
//
// The products of one cell are added in ascending k with fused
// multiply-adds, exactly as in the naive kernel, so the two give identical
// results ("Tiled Matrix Multiplication in CUDA", section 8).

#include "gemm_internal.h"

namespace gemm_f32_impl {
namespace {

template <int T, int PAD>
__global__ __launch_bounds__(T * T) void gemm_lds_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n, BatchArgs bt) {
    __shared__ float tileA[T][T + PAD];
    __shared__ float tileB[T][T + PAD];

    const int tx = threadIdx.x, ty = threadIdx.y;
    const int tile = batch_select(blockIdx.x, tiles_m * tiles_n, bt, A, B, C, K);
    const int tile_row = tile / tiles_n;
    const int tile_col = tile - tile_row * tiles_n;
    const int row = tile_row * T + ty;
    const int col = tile_col * T + tx;
    const bool row_ok = row < M, col_ok = col < N;
    const float *a_row = A + static_cast<int64_t>(row_ok ? row : 0) * lda;

    float acc = 0.0f;
    const int phases = (K + T - 1) / T;
    for (int phase = 0; phase < phases; ++phase) {
        const int a_col = phase * T + tx;  // A walks right
        const int b_row = phase * T + ty;  // B walks down
        tileA[ty][tx] = (row_ok && a_col < K) ? a_row[a_col] : 0.0f;
        tileB[ty][tx] = (b_row < K && col_ok) ? B[static_cast<int64_t>(b_row) * ldb + col] : 0.0f;
        __syncthreads();  // read after write: the whole tile is in LDS

#pragma unroll
        for (int k = 0; k < T; ++k) acc = fmaf(tileA[ty][k], tileB[k][tx], acc);
        __syncthreads();  // write after read: nobody still reads this tile
    }
    if (row_ok && col_ok) C[static_cast<int64_t>(row) * ldc + col] = acc;
}

template <int T, int PAD>
hipError_t launch_lds(const Problem &p, hipStream_t stream) {
    if (p.ta || p.tb) return hipErrorNotSupported;
    const int tiles_n = ceil_div(p.N, T);
    const int tiles_m = ceil_div(p.M, T);
    const int64_t grid = static_cast<int64_t>(tiles_n) * tiles_m * p.batch;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_lds_kernel<T, PAD>), dim3(static_cast<unsigned>(grid)), dim3(T, T),
                       0, stream, p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m,
                       tiles_n, batch_of(p));
    return hipGetLastError();
}

const ConfigEntry kLdsConfigs[] = {
    {"lds_t16", launch_lds<16, 0>, 0},
    {"lds_t32", launch_lds<32, 0>, 0},
    {"lds_t16_pad1", launch_lds<16, 1>, 0},
    {"lds_t32_pad1", launch_lds<32, 1>, 0},
};

}  // namespace

const ConfigEntry *lds_configs(int *count) {
    *count = static_cast<int>(sizeof(kLdsConfigs) / sizeof(kLdsConfigs[0]));
    return kLdsConfigs;
}

}  // namespace gemm_f32_impl
