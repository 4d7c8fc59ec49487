// Stage 4: FP32 matrix cores (MFMA) with double-buffered LDS staging.
//
// Same blocking as the earlier stages -- a workgroup owns a BM x BN tile of
// C and walks K in steps of BK through LDS ("Tiled GEMM: Matrix
// Multiplication in CUDA", section 2) -- with three changes for CDNA4:
//
//  * The inner product runs on v_mfma_f32_32x32x2_f32: one instruction adds
//    a 32 x 2 slice of A times a 2 x 32 slice of B into a 32 x 32 FP32
//    accumulator block held in 16 registers per lane.  Each wavefront owns a
//    (BM / WM) x (BN / WN) sub-tile, i.e. FM x FN accumulator blocks: the
//    register patch of "Tiling and Blocking for Reuse" ("the next level:
//    register blocking"), at wavefront granularity.
//  * Double buffering ("Tiled GEMM: Matrix Multiplication in CUDA",
//    section 8): the global loads of K-step t + 1 go into registers before
//    the matrix-core work of step t, and land in the other LDS buffer after
//    it.  One barrier per K-step then covers both hazards of the two-barrier
//    scheme (sections 4.5 and 4.7 of the same page): the buffer written in
//    step t is read only after the barrier that ends step t, and the buffer
//    read in step t is overwritten only in step t + 1, after that barrier.
//  * Edge tiles ("Tiled GEMM: Matrix Multiplication in CUDA", section 7.1):
//    out-of-range elements of A and B are loaded as 0.0 and the stores are
//    guarded; shapes that are tile multiples compile without the checks.
//
// Operand layout.  For the 32x32x2 instruction lane l supplies A[l % 32][kk]
// and B[kk][l % 32] with kk = l / 32, and accumulator register r of lane l
// holds row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32.  Within a
// chunk of 8 k values the kernel feeds instruction s (s = 0..3) with
// k = 4 * kk + s, a fixed permutation of the chunk applied to A and B alike,
// so lane l needs the 4 consecutive values A[m][4 * kk .. 4 * kk + 3]: one
// 16-byte LDS read per accumulator row block serves 4 instructions.  B is
// read as single floats, 32 consecutive columns per half wavefront.
//
// LDS padding ("Tiled GEMM: Matrix Multiplication in CUDA", section 7.2):
// rows of the A tile are BK floats; lanes 0..31 read 16 bytes each from 32
// consecutive rows, which at BK = 16 would put every second lane in the same
// banks.  PADA = 4 floats of padding shifts consecutive rows by 80 bytes and
// the 16-byte reads of any 8 (or 16) consecutive lanes then fall into
// disjoint banks.  PADB pads the B rows for the same reason when the two
// half wavefronts read rows 4 apart.
//
// Roofline: MFMA bound (compulsory arithmetic intensity of a 256 x 256 x K
// tile is 64 FLOP per byte of A and B, above the 19.7 FLOP/B balance point of
// MI355X's 157.3 TFLOP/s FP32 matrix peak and 8 TB/s HBM).

#include "gemm_internal.h"

namespace gemm_f32_impl {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

// Four consecutive floats of one row starting at column `col`: a 16-byte load
// when the row is 16-byte aligned (VEC), zeros outside [0, limit) and for
// rows that do not exist (GUARD).
template <bool GUARD, bool VEC>
__device__ __forceinline__ float4 load_row4(const float *row_ptr, int col, int limit, bool row_ok) {
    if constexpr (!GUARD) {
        if constexpr (VEC) return *reinterpret_cast<const float4 *>(row_ptr + col);
        return make_float4(row_ptr[col], row_ptr[col + 1], row_ptr[col + 2], row_ptr[col + 3]);
    } else {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row_ok) {
            if (VEC && col + 3 < limit) {
                v = *reinterpret_cast<const float4 *>(row_ptr + col);
            } else {
                if (col + 0 < limit) v.x = row_ptr[col + 0];
                if (col + 1 < limit) v.y = row_ptr[col + 1];
                if (col + 2 < limit) v.z = row_ptr[col + 2];
                if (col + 3 < limit) v.w = row_ptr[col + 3];
            }
        }
        return v;
    }
}

template <int BM, int BN, int BK, int WM, int WN, int PADA, int PADB, bool GUARD, bool VEC>
__global__ __launch_bounds__(64 * WM * WN) void gemm_mfma_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n, int group_m) {
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;  // wavefront sub-tile
    constexpr int FM = WTM / 32, FN = WTN / 32;  // 32 x 32 blocks per wavefront
    constexpr int LA = (BM * BK) / (4 * NT);     // float4 loads of A per thread
    constexpr int LB = (BK * BN) / (4 * NT);     // float4 loads of B per thread
    constexpr int LDA_S = BK + PADA, LDB_S = BN + PADB;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is whole 32 x 32 blocks");
    static_assert(BK % 8 == 0, "K step is whole chunks of 8");
    static_assert(LA * 4 * NT == BM * BK && LB * 4 * NT == BK * BN, "even tile split");
    static_assert(LDA_S % 4 == 0 && LDB_S % 4 == 0, "16-byte aligned LDS rows");

    __shared__ __align__(16) float sA[2][BM * LDA_S];  // m-major, k contiguous
    __shared__ __align__(16) float sB[2][BK * LDB_S];  // k-major, n contiguous

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    int tm, tn;
    grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // Per-thread global load slots (fixed across K-steps).
    int a_m[LA], a_k[LA], b_k[LB], b_n[LB];
    const float *a_row[LA];
    bool a_ok[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int e = tid + i * NT;
        a_m[i] = e / (BK / 4);
        a_k[i] = (e % (BK / 4)) * 4;
        const int gm = m0 + a_m[i];
        a_ok[i] = gm < M;
        a_row[i] = A + static_cast<int64_t>(a_ok[i] ? gm : 0) * lda;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int e = tid + i * NT;
        b_k[i] = e / (BN / 4);
        b_n[i] = (e % (BN / 4)) * 4;
    }

    float4 ra[LA], rb[LB];
    auto load_global = [&](int k0) {
#pragma unroll
        for (int i = 0; i < LA; ++i)
            ra[i] = load_row4<GUARD, VEC>(a_row[i], k0 + a_k[i], K, a_ok[i]);
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            const int gk = k0 + b_k[i];
            const bool ok = !GUARD || gk < K;
            const float *row = B + static_cast<int64_t>(ok ? gk : 0) * ldb + n0;
            rb[i] = load_row4<GUARD, VEC>(row, b_n[i], N - n0, ok);
        }
    };
    auto store_lds = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LA; ++i)
            *reinterpret_cast<float4 *>(&sA[buf][a_m[i] * LDA_S + a_k[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < LB; ++i)
            *reinterpret_cast<float4 *>(&sB[buf][b_k[i] * LDB_S + b_n[i]]) = rb[i];
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int half = lane >> 5;  // kk of this lane
    const int l32 = lane & 31;
    const int a_lds = (wm * WTM + l32) * LDA_S + 4 * half;
    const int b_lds = (4 * half) * LDB_S + wn * WTN + l32;

    const int nk = (K + BK - 1) / BK;
    load_global(0);
    store_lds(0);
    __syncthreads();

    for (int t = 0; t < nk; ++t) {
        const int buf = t & 1;
        if (t + 1 < nk) load_global((t + 1) * BK);

        const float *pa = &sA[buf][a_lds];
        const float *pb = &sB[buf][b_lds];
#pragma unroll
        for (int kc = 0; kc < BK / 8; ++kc) {
            float4 af[FM];
            float bf[FN][4];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const float4 *>(pa + i * 32 * LDA_S + kc * 8);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int s = 0; s < 4; ++s) bf[j][s] = pb[(kc * 8 + s) * LDB_S + j * 32];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const float a = s == 0 ? af[i].x : s == 1 ? af[i].y : s == 2 ? af[i].z : af[i].w;
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bf[j][s], acc[i][j], 0, 0, 0);
                    }
        }

        if (t + 1 < nk) store_lds(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: accumulator register r of lane l is row
    //      8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32 of its block ----
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int gn = n0 + wn * WTN + j * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm * WTM + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                if (!GUARD || (gm < M && gn < N))
                    C[static_cast<int64_t>(gm) * ldc + gn] = acc[i][j][r];
            }
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int PADA, int PADB, int GROUP_M>
hipError_t launch_mfma(const Problem &p, hipStream_t stream) {
    constexpr int NT = 64 * WM * WN;
    const int tiles_m = ceil_div(p.M, BM), tiles_n = ceil_div(p.N, BN);
    const int64_t grid = static_cast<int64_t>(tiles_m) * tiles_n;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool vec = rows_aligned16(p.A, p.lda) && rows_aligned16(p.B, p.ldb);
    const bool guard = (p.M % BM) || (p.N % BN) || (p.K % BK);
    const dim3 g(static_cast<unsigned>(grid)), b(NT);
#define GEMM_MFMA_LAUNCH(G, V)                                                                 \
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, WM, WN, PADA, PADB, G, V>), g, b, 0, stream, \
                       p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n, GROUP_M)
    if (guard) {
        if (vec) GEMM_MFMA_LAUNCH(true, true);
        else GEMM_MFMA_LAUNCH(true, false);
    } else {
        if (vec) GEMM_MFMA_LAUNCH(false, true);
        else GEMM_MFMA_LAUNCH(false, false);
    }
#undef GEMM_MFMA_LAUNCH
    return hipGetLastError();
}

const ConfigEntry kMfmaConfigs[] = {
    {"mfma_128x128x16_w2x2_pa4_pb0", launch_mfma<128, 128, 16, 2, 2, 4, 0, 8>, 128, 128, 16},
    {"mfma_128x128x16_w2x2_pa0_pb0", launch_mfma<128, 128, 16, 2, 2, 0, 0, 8>, 128, 128, 16},
    {"mfma_128x128x16_w2x2_pa4_pb8", launch_mfma<128, 128, 16, 2, 2, 4, 8, 8>, 128, 128, 16},
    {"mfma_128x128x32_w2x2_pa4_pb0", launch_mfma<128, 128, 32, 2, 2, 4, 0, 8>, 128, 128, 32},
    {"mfma_256x128x16_w2x2_pa4_pb0", launch_mfma<256, 128, 16, 2, 2, 4, 0, 8>, 256, 128, 16},
    {"mfma_128x256x16_w2x2_pa4_pb0", launch_mfma<128, 256, 16, 2, 2, 4, 0, 8>, 128, 256, 16},
    {"mfma_256x256x16_w2x2_pa4_pb0", launch_mfma<256, 256, 16, 2, 2, 4, 0, 8>, 256, 256, 16},
    {"mfma_256x256x16_w2x4_pa4_pb0", launch_mfma<256, 256, 16, 2, 4, 4, 0, 8>, 256, 256, 16},
    {"mfma_64x64x16_w2x2_pa4_pb0", launch_mfma<64, 64, 16, 2, 2, 4, 0, 8>, 64, 64, 16},
    {"mfma_64x64x32_w2x2_pa4_pb0", launch_mfma<64, 64, 32, 2, 2, 4, 0, 8>, 64, 64, 32},
};

}  // namespace

const ConfigEntry *mfma_configs(int *count) {
    *count = static_cast<int>(sizeof(kMfmaConfigs) / sizeof(kMfmaConfigs[0]));
    return kMfmaConfigs;
}

}  // namespace gemm_f32_impl
