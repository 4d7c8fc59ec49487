// Stage 2: the K dimension in T-wide phases through LDS.
//
// Prior art: the shared-memory tiled kernels of "Tiled Matrix Multiplication
// in CUDA" (section 7) and "Tiled GEMM: Matrix Multiplication in CUDA"
// (sections 2 and 4).  This stage is that method by design, so the steps
// match the pages' (copy, barrier, partial dot products, barrier); the code
// below is its own.
//
// One T x T workgroup owns one T x T block of C, a lane per cell.  For each
// phase of T values of k the workgroup first copies the T x T block of A
// (C's rows, the phase's k) and the T x T block of B (the phase's k, C's
// columns) into LDS, one element of each per lane, and waits: every lane
// then finds all T of its A values and T of its B values in LDS.  Each lane
// adds its T products, and the workgroup waits again before the next phase
// overwrites the blocks.  An element loaded from global memory serves T
// lanes, so requested traffic falls by T against the naive kernel and the
// intensity becomes T / 4 FLOP per byte ("Tiled GEMM: Matrix Multiplication
// in CUDA", section 2).
//
// Ragged shapes ("Tiled GEMM: Matrix Multiplication in CUDA", section 7.1):
// blocks that reach past M, N or K are padded with zeros in LDS, which add
// nothing to any sum, and only cells inside C are stored.
//
// LDS banks (section 7.2 of the same page): in the product loop all lanes
// of a row read one A value (a broadcast) and consecutive lanes read
// consecutive B values, so no padding is needed; PAD = 1 builds exist to
// show that in the bank-conflict counters.
//
// Each cell's products are added in ascending k with fused multiply-adds,
// the order of the naive kernel, so both stages return the same bits
// ("Tiled Matrix Multiplication in CUDA", section 8).

#include "gemm_internal.h"

namespace gemm_f32_impl {
namespace {

template <int T, int PAD>
__global__ __launch_bounds__(T * T) void gemm_lds_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n, BatchArgs bt) {
    // s_a[r][q]: A at (block row r, phase k q); s_b[q][c]: B at (phase k q,
    // block column c)
    __shared__ float s_a[T][T + PAD];
    __shared__ float s_b[T][T + PAD];

    const int lx = threadIdx.x;  // cell column in the block; k offset of the A copy
    const int ly = threadIdx.y;  // cell row in the block; k offset of the B copy
    const int blk = batch_select(blockIdx.x, tiles_m * tiles_n, bt, A, B, C, K);
    const int bi = blk / tiles_n, bj = blk - (blk / tiles_n) * tiles_n;
    const int i = bi * T + ly, j = bj * T + lx;  // this lane's cell of C
    const bool in_m = i < M, in_n = j < N;

    // The elements this lane copies in phase p: A(i, pT + lx) and
    // B(pT + ly, j).  Both pointers advance by one phase per iteration.
    const float *pa = A + static_cast<int64_t>(in_m ? i : 0) * lda + lx;
    const float *pb = B + static_cast<int64_t>(ly) * ldb + (in_n ? j : 0);
    const int64_t pb_step = static_cast<int64_t>(T) * ldb;

    float sum = 0.0f;
    for (int k0 = 0; k0 < K; k0 += T) {
        s_a[ly][lx] = (in_m && k0 + lx < K) ? *pa : 0.0f;
        s_b[ly][lx] = (in_n && k0 + ly < K) ? *pb : 0.0f;
        pa += T;
        pb += pb_step;
        __syncthreads();  // both blocks are complete in LDS

#pragma unroll
        for (int q = 0; q < T; ++q) sum = fmaf(s_a[ly][q], s_b[q][lx], sum);
        __syncthreads();  // no lane still reads them when the next phase writes
    }
    if (in_m && in_n) C[static_cast<int64_t>(i) * ldc + j] = sum;
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
