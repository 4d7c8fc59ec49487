// Internal declarations shared by the HIP kernels and the C-ABI layer of
// libgemm_f32.so.  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gemm_f32_impl {

// One validated problem: C (M x N, ldc) = A (M x K, lda) x B (K x N, ldb),
// all row-major ("Tiled Matrix Multiplication in CUDA", section 2;
// "Tiled GEMM: Matrix Multiplication in CUDA", section 7.1).  Sizes fit in
// int after validation; leading dimensions stay 64-bit so that row offsets
// are formed in 64-bit arithmetic.
struct Problem {
    int M, N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    float *C;
    int64_t ldc;
    // Independent products C_b = A_b x B_b, b < batch, with X_b = X + b * sX
    // (one product: batch 1, strides 0).
    int batch;
    int64_t sa, sb, sc;
    // Transposed operands: op(A) = A^T with A stored K x M (row-major, lda),
    // op(B) = B^T with B stored N x K (ldb).
    bool ta, tb;
    // Split-K partial products: product b covers k in [b * ksplit,
    // min((b + 1) * ksplit, K)) (0: every product runs over all of K).
    int ksplit;
};

// Batch description passed to the kernels.
struct BatchArgs {
    int count;
    int64_t sa, sb, sc;
    int ksplit;
};
inline BatchArgs batch_of(const Problem &p) { return {p.batch, p.sa, p.sb, p.sc, p.ksplit}; }

// Host-side launch of one tile configuration.  Returns hipSuccess or the
// error of the launch.
using LaunchFn = hipError_t (*)(const Problem &, hipStream_t);

// Capabilities of a configuration beyond plain row-major operands.
constexpr unsigned kCapTransposed = 1u;  // accepts transposed A and/or B

struct ConfigEntry {
    const char *name;  // stable, used by the tuning table and benchmarks
    LaunchFn launch;
    unsigned caps;
};

// Registries, one per variant (defined in the kernel sources).
const ConfigEntry *naive_configs(int *count);
const ConfigEntry *lds_configs(int *count);
const ConfigEntry *regblock_configs(int *count);
const ConfigEntry *mfma_configs(int *count);    // all MFMA configurations
const ConfigEntry *mfma16_configs(int *count);  // those with 16x16x4 instructions
const ConfigEntry *mfma_regs_configs(int *count);  // operands loaded straight into registers

// Sets the C region to zero (the K == 0 case).  A fill kernel rather than a
// memset so that a captured graph replays it faithfully and ldc padding is
// never touched.
hipError_t launch_zero_fill(float *C, int M, int N, int64_t ldc, int batch, int64_t sc,
                            hipStream_t stream);

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// 16-byte alignment of a base pointer, a leading dimension and a batch
// stride: float4 loads along a row are then aligned for every row of every
// product.
inline bool rows_aligned16(const float *p, int64_t ld, int64_t stride = 0) {
    return (reinterpret_cast<uintptr_t>(p) % 16u) == 0 && (ld % 4) == 0 && (stride % 4) == 0;
}

}  // namespace gemm_f32_impl

// --------------------------------------------------------------------------
// Device helpers
// --------------------------------------------------------------------------

// Workgroups of one launch are handed to the 8 XCDs of an MI355X in
// round-robin order (workgroup b runs on XCD b % 8), and each XCD has its own
// L2.  This maps the hardware order to a "logical" order in which
// consecutive ids sit on the same XCD, so that tiles which share rows of A or
// columns of B also share an L2.  The map is a bijection on [0, n) for any n.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    constexpr int kXcds = 8;
    const int q = n / kXcds, r = n % kXcds;
    const int xcd = bid % kXcds, local = bid / kXcds;
    return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Splits a linear workgroup id over `tiles` tiles per product into the
// product index (applied to the three base pointers, and for split-K
// partial products to the K extent) and the tile index.
template <class PA, class PB, class PC>
__device__ __forceinline__ int batch_select(int lin, int tiles, const gemm_f32_impl::BatchArgs &bt,
                                            PA &A, PB &B, PC &C, int &K) {
    const int b = lin / tiles;
    A += static_cast<int64_t>(b) * bt.sa;
    B += static_cast<int64_t>(b) * bt.sb;
    C += static_cast<int64_t>(b) * bt.sc;
    if (bt.ksplit > 0) K = min(bt.ksplit, K - b * bt.ksplit);
    return lin - b * tiles;
}

// Grouped ordering of output tiles: consecutive logical ids walk down a
// column strip of `group_m` tile rows before moving right, so a run of
// workgroups reuses the same B columns and a small set of A rows.
__device__ __forceinline__ void grouped_tile(int id, int tiles_m, int tiles_n, int group_m,
                                             int &tm, int &tn) {
    const int per_group = group_m * tiles_n;
    const int group = id / per_group;
    const int first_m = group * group_m;
    const int rows = min(tiles_m - first_m, group_m);
    const int in_group = id - group * per_group;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}
