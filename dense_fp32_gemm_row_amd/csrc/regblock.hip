// Stage 3: register blocking on the vector ALUs.
//
// Prior art: "Tiling and Blocking for Reuse", "the next level: register
// blocking".  Every thread owns a TM x TN patch of C in registers.  Per k it
// reads TM values of the A tile and TN values of the B tile from LDS and
// performs TM * TN multiply-adds with them, so LDS reads per multiply-add
// fall from 2 (one of them a broadcast) in the tiled kernel to
// (TM + TN) / (TM * TN): 1/2 for the page's 4 x 4 patch, 1/4 for 8 x 8.
// Register pressure, not LDS, now bounds the patch size (same section).
//
// Workgroup: (BM / TM) x (BN / TN) threads computing a BM x BN tile of C,
// K walked in steps of BK with the two barriers of the tiled kernel.
//
// LDS layout.  The A tile is stored k-major, tileA[k][m], so that a thread
// reads its TM values of one k as float4 vectors; the global reads of A run
// along k, so the store into LDS is a transpose.  Consecutive lanes then write
// the same column m of consecutive rows k, which with a row length that is a
// multiple of the bank count puts them all in one bank.  Padding each LDS row
// by PAD floats moves consecutive rows to different banks -- the padded
// transposed tile of "Tiled GEMM: Matrix Multiplication in CUDA", section 7.2.
// The pad is 4 floats rather than 1 so that rows stay 16-byte aligned for the
// vector reads; PAD = 0 configurations exist to compare the counters.
//
// Thread patch.  The TM x TN patch is split into 4 x 4 sub-blocks spread
// across the tile at strides of 4 * (threads per dimension), so the float4
// reads of the 16 threads along a row of the thread grid cover 256 contiguous
// bytes of LDS and the 4 rows of threads in a wavefront share them by
// broadcast.
//
// The products of one cell are added in ascending k with fused
// multiply-adds, as in the naive and tiled kernels, so all three give
// identical results.

#include "gemm_internal.h"

namespace gemm_f32_impl {
namespace {

template <int BM, int BN, int BK, int TM, int TN, int PAD, bool VEC>
__global__ __launch_bounds__((BM / TM) * (BN / TN)) void gemm_regblock_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n, BatchArgs bt, bool vec_store) {
    constexpr int TX = BN / TN;  // threads along columns
    constexpr int TY = BM / TM;  // threads along rows
    constexpr int NT = TX * TY;
    constexpr int SM = 4 * TY;   // row stride between a thread's 4 x 4 sub-blocks
    constexpr int SN = 4 * TX;   // column stride between them
    static_assert(TM % 4 == 0 && TN % 4 == 0, "patch is built from 4 x 4 sub-blocks");
    static_assert((BM * BK) % (4 * NT) == 0 && (BK * BN) % (4 * NT) == 0, "even tile split");
    static_assert((BM + PAD) % 4 == 0 && (BN + PAD) % 4 == 0, "16-byte aligned LDS rows");

    __shared__ __align__(16) float tileA[BK][BM + PAD];  // k-major (transposed)
    __shared__ __align__(16) float tileB[BK][BN + PAD];  // k-major (as in memory)

    const int tid = threadIdx.x;
    const int tx = tid % TX, ty = tid / TX;
    int tm, tn;
    const int tile = batch_select(xcd_remap(blockIdx.x, tiles_m * tiles_n * bt.count),
                                  tiles_m * tiles_n, bt, A, B, C, K);
    grouped_tile(tile, tiles_m, tiles_n, 8, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += BK) {
        // ---- cooperative load of the A tile (BM x BK), zero outside A ----
        if constexpr (VEC) {
#pragma unroll
            for (int i = 0; i < (BM * BK) / (4 * NT); ++i) {
                const int e = tid + i * NT;
                const int m = e / (BK / 4), kq = (e % (BK / 4)) * 4;
                const int gm = m0 + m, gk = k0 + kq;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (gm < M) {
                    const float *src = A + static_cast<int64_t>(gm) * lda + gk;
                    if (gk + 3 < K) {
                        v = *reinterpret_cast<const float4 *>(src);
                    } else {
                        v.x = gk + 0 < K ? src[0] : 0.f;
                        v.y = gk + 1 < K ? src[1] : 0.f;
                        v.z = gk + 2 < K ? src[2] : 0.f;
                    }
                }
                tileA[kq + 0][m] = v.x;
                tileA[kq + 1][m] = v.y;
                tileA[kq + 2][m] = v.z;
                tileA[kq + 3][m] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < (BM * BK) / NT; ++i) {
                const int e = tid + i * NT;
                const int m = e / BK, k = e % BK;
                const int gm = m0 + m, gk = k0 + k;
                tileA[k][m] = (gm < M && gk < K) ? A[static_cast<int64_t>(gm) * lda + gk] : 0.f;
            }
        }
        // ---- cooperative load of the B tile (BK x BN), zero outside B ----
        if constexpr (VEC) {
#pragma unroll
            for (int i = 0; i < (BK * BN) / (4 * NT); ++i) {
                const int e = tid + i * NT;
                const int k = e / (BN / 4), nq = (e % (BN / 4)) * 4;
                const int gk = k0 + k, gn = n0 + nq;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (gk < K) {
                    const float *src = B + static_cast<int64_t>(gk) * ldb + gn;
                    if (gn + 3 < N) {
                        v = *reinterpret_cast<const float4 *>(src);
                    } else {
                        v.x = gn + 0 < N ? src[0] : 0.f;
                        v.y = gn + 1 < N ? src[1] : 0.f;
                        v.z = gn + 2 < N ? src[2] : 0.f;
                    }
                }
                *reinterpret_cast<float4 *>(&tileB[k][nq]) = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < (BK * BN) / NT; ++i) {
                const int e = tid + i * NT;
                const int k = e / BN, n = e % BN;
                const int gk = k0 + k, gn = n0 + n;
                tileB[k][n] = (gk < K && gn < N) ? B[static_cast<int64_t>(gk) * ldb + gn] : 0.f;
            }
        }
        __syncthreads();  // read after write

#pragma unroll
        for (int k = 0; k < BK; ++k) {
            float a[TM], b[TN];
#pragma unroll
            for (int p = 0; p < TM / 4; ++p) {
                const float4 v = *reinterpret_cast<const float4 *>(&tileA[k][p * SM + ty * 4]);
                a[p * 4 + 0] = v.x; a[p * 4 + 1] = v.y; a[p * 4 + 2] = v.z; a[p * 4 + 3] = v.w;
            }
#pragma unroll
            for (int q = 0; q < TN / 4; ++q) {
                const float4 v = *reinterpret_cast<const float4 *>(&tileB[k][q * SN + tx * 4]);
                b[q * 4 + 0] = v.x; b[q * 4 + 1] = v.y; b[q * 4 + 2] = v.z; b[q * 4 + 3] = v.w;
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();  // write after read
    }

    // ---- epilogue: guarded stores of the patch ----
#pragma unroll
    for (int p = 0; p < TM / 4; ++p) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int gm = m0 + p * SM + ty * 4 + r;
            if (gm >= M) continue;
            float *crow = C + static_cast<int64_t>(gm) * ldc;
#pragma unroll
            for (int q = 0; q < TN / 4; ++q) {
                const int gn = n0 + q * SN + tx * 4;
                const float *v = &acc[p * 4 + r][q * 4];
                if (vec_store && gn + 3 < N) {
                    *reinterpret_cast<float4 *>(crow + gn) = make_float4(v[0], v[1], v[2], v[3]);
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (gn + c < N) crow[gn + c] = v[c];
                }
            }
        }
    }
}

template <int BM, int BN, int BK, int TM, int TN, int PAD>
hipError_t launch_regblock(const Problem &p, hipStream_t stream) {
    if (p.ta || p.tb) return hipErrorNotSupported;
    constexpr int NT = (BM / TM) * (BN / TN);
    const int tiles_m = ceil_div(p.M, BM), tiles_n = ceil_div(p.N, BN);
    const int64_t grid = static_cast<int64_t>(tiles_m) * tiles_n * p.batch;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool vec = rows_aligned16(p.A, p.lda, p.sa) && rows_aligned16(p.B, p.ldb, p.sb);
    const bool vec_store = rows_aligned16(p.C, p.ldc, p.sc);
    if (vec)
        hipLaunchKernelGGL((gemm_regblock_kernel<BM, BN, BK, TM, TN, PAD, true>),
                           dim3(static_cast<unsigned>(grid)), dim3(NT), 0, stream, p.M, p.N,
                           p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n, batch_of(p),
                           vec_store);
    else
        hipLaunchKernelGGL((gemm_regblock_kernel<BM, BN, BK, TM, TN, PAD, false>),
                           dim3(static_cast<unsigned>(grid)), dim3(NT), 0, stream, p.M, p.N,
                           p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n, batch_of(p),
                           vec_store);
    return hipGetLastError();
}

const ConfigEntry kRegblockConfigs[] = {
    {"regblock_128x128x8_t8x8_pad4", launch_regblock<128, 128, 8, 8, 8, 4>, 0},
    {"regblock_64x64x16_t4x4_pad4", launch_regblock<64, 64, 16, 4, 4, 4>, 0},
    {"regblock_128x128x8_t8x8_pad0", launch_regblock<128, 128, 8, 8, 8, 0>, 0},
    {"regblock_128x128x16_t8x8_pad4", launch_regblock<128, 128, 16, 8, 8, 4>, 0},
    {"regblock_128x64x16_t8x4_pad4", launch_regblock<128, 64, 16, 8, 4, 4>, 0},
};

}  // namespace

const ConfigEntry *regblock_configs(int *count) {
    *count = static_cast<int>(sizeof(kRegblockConfigs) / sizeof(kRegblockConfigs[0]));
    return kRegblockConfigs;
}

}  // namespace gemm_f32_impl
