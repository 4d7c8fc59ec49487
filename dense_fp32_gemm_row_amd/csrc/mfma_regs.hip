// MFMA tiles whose operands go from global memory straight into registers.
//
// With about one output tile per CU the LDS-staged kernels spend a good
// share of every K-step on the LDS round trip and the barrier that ends it
// (a sixth for the 64 x 64 k-group tile of the ragged 1000 x 1023 x 777
// shape).  Here each wavefront loads the MFMA operands it needs itself, in
// the register layout the instruction takes, a few chunks of 16 k ahead: no
// LDS stores, no LDS reads and no barrier in the K loop.  LDS serves only
// the sum of the k-groups' partial tiles at the end.
//
// Blocking ("Tiled GEMM: Matrix Multiplication in CUDA", section 2): a
// workgroup owns a BM x BN tile of C; KG k-groups of WM x WN wavefronts split
// K between them in chunks of 16 (chunk c goes to group c mod KG), and each
// wavefront of a group accumulates a (BM / WM) x (BN / WN) slice for its
// chunks in 16 x 16 blocks of v_mfma_f32_16x16x4_f32 (FM x FN blocks).  The
// configurations use one wavefront per group (WM = WN = 1), which owns the
// whole tile, so no operand is loaded twice in a workgroup; one wavefront
// per SIMD leaves 512 registers per lane (256 accumulator floats for
// 128 x 128).  The partial tiles are then added in LDS in group order, a
// fixed order, and stored ("Tiled Matrix Multiplication in CUDA", section
// 5: one final write per output element).
//
// Operand layout of one chunk of 16 k.  Lane l = 16 g + i supplies, to
// instruction s (s = 0..3), op(A)[row][4 g + s] and op(B)[4 g + s][col]: a
// fixed permutation of the chunk applied to A and B alike.  An operand
// stored with k contiguous (A as stored, B transposed) gives a lane its 4
// values of a block in one 16-byte load; one stored k-major (B as stored, A
// transposed) gives it its F interleaved blocks' values of one k row in one
// load of 4 F bytes (see RegOperand).
//
// Edges ("Tiled GEMM: Matrix Multiplication in CUDA", section 7.1).  The K
// loop runs the chunks that hold neither a k past K nor the last k of the
// operand, with clamped addresses and no per-element checks: a row past M
// or N loads the last row, a k-major group that starts past the extent
// loads the group that holds the last row, and a group that starts inside
// it loads as it is (its floats past the extent come from the row's padding
// or the next k row, which exists inside the loop).  Those values only feed
// outputs that are never stored.  The chunk that holds the last k, whole or
// partial, is a tail with zero fill past K, M and N, loaded before the loop
// and split over the groups by instruction.  Shapes where a k-major group
// can reach past the operand's storage even so (an extent below F - 1) run
// a variant that checks every element.  Stores are guarded.
//
// A persistent form of the kernel (one workgroup per CU walking its tiles,
// each tile's last chunks loading the next tile's first ones) serves whole
// tiles with K a multiple of 16 KG D, in every operand form, and in an edge
// form the other shapes whose K and k-major row lengths are multiples of 4
// (positions past M, N or K read zeros: their buffer offset lies past the
// resource).  It loads the operands as buffers (a scalar resource per chunk,
// a lane offset fixed per tile, a scalar offset per k row: no vector address
// arithmetic), each piece right after the last instruction that reads the
// registers it refills.
//
// Roofline: MFMA bound per chunk (4 FM FN instructions of 32 cycles per
// FM + 4 loads, or fewer); the tile's fixed cost (first loads, the k-group
// sum, the stores) is what a short K exposes.

#include <type_traits>

#include "mfma_kernels.h"

// Buffer loads of 16 and 8 bytes: the resource's base plus a lane offset
// (bytes, plus the instruction's constant offset) plus a scalar offset.
__device__ gemm_f32_impl::floatx4 gemm_f32_buffer_load_x4(__amdgpu_buffer_rsrc_t rsrc, int voffset,
                                                          int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.load.v4f32");
__device__ float __attribute__((ext_vector_type(2))) gemm_f32_buffer_load_x2(
    __amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.load.v2f32");

namespace gemm_f32_impl {
namespace {

typedef float floatx2 __attribute__((ext_vector_type(2)));

// N consecutive floats at q (4-byte alignment): one load of 4 N bytes per
// 16-byte piece, which global memory accepts at any 4-byte alignment.
template <int N>
__device__ __forceinline__ void load_run(const float *q, float (&v)[N]) {
    static_assert(N == 1 || N % 2 == 0, "runs of 1 or an even number of floats");
#pragma unroll
    for (int p = 0; p + 4 <= N; p += 4) {
        const floatx4 t = floatx4{q[p], q[p + 1], q[p + 2], q[p + 3]};
        v[p] = t[0], v[p + 1] = t[1], v[p + 2] = t[2], v[p + 3] = t[3];
    }
    if constexpr (N % 4 == 2) {  // the last two: one 8-byte load
        const floatx2 t = floatx2{q[N - 2], q[N - 1]};
        v[N - 2] = t[0], v[N - 1] = t[1];
    } else if constexpr (N == 1) {
        v[0] = q[0];
    }
}
template <int N>
__device__ __forceinline__ void store_run(float *q, const float (&v)[N]) {
    if constexpr (N >= 4) {
#pragma unroll
        for (int p = 0; p < N; p += 4)
            *reinterpret_cast<floatx4 *>(q + p) = floatx4{v[p], v[p + 1], v[p + 2], v[p + 3]};
    } else if constexpr (N == 2) {
        *reinterpret_cast<floatx2 *>(q) = floatx2{v[0], v[1]};
    } else {
        q[0] = v[0];
    }
}

// Rows (f, r) of a wavefront's slice that one pass of the k-group sum
// handles: a multiple of KG that divides FM x 4, as many as LDS holds.
constexpr int regs_pass_rows(int FM, int FN, int KG, int NWG) {
    int best = 0;
    for (int rp = KG; rp <= FM * 4; rp += KG)
        if ((FM * 4) % rp == 0 && KG * NWG * rp * 64 * FN * 4 <= kLdsBytes) best = rp;
    return best;
}

// One operand of a wavefront's slice: F blocks of 16 rows (of op(A)) or
// columns (of op(B)), for lane i of lane group g; x[f][s] is the value the
// lane feeds to instruction s of a chunk for block f, at k = k0 + 4 g + s.
//  * Row flavour (KMAJOR = false): element (r, k) at X[r ld + k], k
//    contiguous (A as stored, B transposed).  A chunk's 4 values of block f
//    are one 16-byte load.
//  * K-major flavour (KMAJOR = true): element (r, k) at X[k ld + r], r
//    contiguous (B as stored, A transposed).  With interleaved blocks a
//    lane's F values of one k row are adjacent: one load of 4 F bytes per s.
// Block f holds rows base + F i + f (IL, interleaved) or base + 16 f + i.
// CLAMP: rows past R (row flavour) load row R - 1, a k-major group that
// starts past R loads the group that holds row R - 1 (their values feed
// outputs that are never stored).
template <bool KMAJOR, int F, bool IL>
struct RegOperand {
    static_assert(!KMAJOR || IL, "k-major operands are interleaved");
    const float *X;
    int64_t ld;
    int r0, R;                 // first row of the lane's group (or block 0), rows of the operand
    const float *p[KMAJOR ? 1 : F];

    __device__ __forceinline__ int row(int base, int i, int f) const {
        return IL ? base + F * i + f : base + 16 * f + i;
    }
    __device__ __forceinline__ void init(const float *X_, int64_t ld_, int R_, int base, int g, int i,
                                         bool clamp) {
        X = X_, ld = ld_, R = R_;
        r0 = row(base, i, 0);
        if constexpr (KMAJOR) {
            const int r = clamp && r0 > R - 1 ? ((R - 1) / F) * F : r0;
            p[0] = X + static_cast<int64_t>(4 * g) * ld + r;
        } else {
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const int rr = row(base, i, f);
                const int r = clamp && rr > R - 1 ? R - 1 : rr;
                p[f] = X + static_cast<int64_t>(r) * ld + 4 * g;
            }
        }
    }
    // chunk c, clamped addresses
    __device__ __forceinline__ void load(float (&x)[F][4], int c) const {
        const int k0 = c * 16;
        if constexpr (KMAJOR) {
            const float *q = p[0] + static_cast<int64_t>(k0) * ld;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                float v[F];
                load_run<F>(q + s * ld, v);
#pragma unroll
                for (int f = 0; f < F; ++f) x[f][s] = v[f];
            }
        } else {
#pragma unroll
            for (int f = 0; f < F; ++f) load_run<4>(p[f] + k0, x[f]);
        }
    }
    // chunk c with zero fill past K and R: vector loads where all of a
    // lane's values are in range, single floats where they straddle K or R
    __device__ __forceinline__ void load_checked(float (&x)[F][4], int c, int g, int K) const {
        const int k0 = c * 16 + 4 * g;
        if constexpr (KMAJOR) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bool ok = k0 + s < K;
                const float *q = X + static_cast<int64_t>(ok ? k0 + s : 0) * ld + r0;
                float v[F];
                if (ok && r0 + F - 1 < R) {
                    load_run<F>(q, v);
                } else {
#pragma unroll
                    for (int f = 0; f < F; ++f) v[f] = ok && r0 + f < R ? q[f] : 0.0f;
                }
#pragma unroll
                for (int f = 0; f < F; ++f) x[f][s] = v[f];
            }
        } else {
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const float *q = p[f] + c * 16;  // row clamped: only unstored outputs see it
                if (k0 + 3 < K) {
                    load_run<4>(q, x[f]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[f][e] = k0 + e < K ? q[e] : 0.0f;
                }
            }
        }
    }
};

// An operand of the persistent kernel, loaded as a buffer: the chunk's
// origin is a scalar resource, a lane's place in the chunk a 32-bit byte
// offset fixed for the tile, and a k row's distance a scalar offset, so a
// load of a whole tile takes no vector address arithmetic.  Same layout and
// lane mapping as RegOperand; a k-major operand's F floats of one k row go
// in 16-byte loads and, for F = 4 n + 2, one 8-byte load.
// Offsets stay below 2^31 bytes: the launcher checks (rows - 1) ld + 16
// (row flavour) and 15 ld + rows (k-major) against 2^28 floats.
// EDGE: rows past R and k past K read as zeros: their offset is 2^31, past
// the resource's 2^31 - 1 bytes, and an out-of-range buffer load returns 0.
// Whole rows (row flavour) or groups of 4 (k-major) are in or out: K, and
// R of a k-major operand, are multiples of 4, and F of a k-major operand
// too (the launcher checks).
template <bool KMAJOR, int F, bool IL, bool EDGE = false>
struct BufOperand {
    static_assert(!KMAJOR || (IL && F % 2 == 0), "k-major operands: interleaved, 16- and 8-byte pieces");
    static_assert(!(KMAJOR && EDGE) || F % 4 == 0, "edge form: k-major groups of 4");
    static constexpr bool kKMajor = KMAJOR;
    static constexpr int kPieces = KMAJOR ? 4 : F;
    static constexpr int kOut = static_cast<int>(0x80000000u);  // an offset past the resource
    const float *X;  // the tile's origin: row r0 (row flavour) or column r0 (k-major), k = 0
    int ld;
    int voff[KMAJOR ? (EDGE ? F / 4 : 1) : F];
    int klim;  // EDGE: K - 4 g, the lane's first k past the operand (relative to the chunk)

    __device__ __forceinline__ void init(const float *X_, int64_t ld_, int base, int g, int i, int R = 0,
                                         int K = 0) {
        ld = static_cast<int>(ld_);
        klim = K - 4 * g;
        if constexpr (KMAJOR) {
            X = X_ + base;
            if constexpr (EDGE) {
#pragma unroll
                for (int p = 0; p < F; p += 4)
                    voff[p / 4] = base + F * i + p < R ? (4 * g * ld + F * i + p) * 4 : kOut;
            } else {
                voff[0] = (4 * g * ld + F * i) * 4;
            }
        } else {
            X = X_ + static_cast<int64_t>(base) * ld_;
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const int r = IL ? F * i + f : 16 * f + i;
                voff[f] = !EDGE || base + r < R ? (r * ld + 4 * g) * 4 : kOut;
            }
        }
    }
    // chunk c's origin: k = 16 c
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk(int c) const {
        const float *o = KMAJOR ? X + static_cast<int64_t>(c * 16) * ld : X + c * 16;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(o), 0, 0x7fffffff, 0x00020000);
    }
    // piece q of chunk c: k row q of a k-major operand (x[.][q]), block q of
    // a row operand (x[q][.]); KCHK: the chunk may hold k past K (a per-lane
    // check, otherwise none)
    template <bool KCHK>
    __device__ __forceinline__ void load_piece(float (&x)[F][4], int c, int q) const {
        constexpr bool kc = EDGE && KCHK;
        const __amdgpu_buffer_rsrc_t rs = chunk(c);
        if constexpr (KMAJOR) {
            const bool kin = !kc || c * 16 + q < klim;
#pragma unroll
            for (int p = 0; p + 4 <= F; p += 4) {
                const int v = EDGE ? voff[p / 4] : voff[0] + 4 * p;
                const floatx4 t = gemm_f32_buffer_load_x4(rs, kin ? v : kOut, q * ld * 4, 0);
                x[p][q] = t[0], x[p + 1][q] = t[1], x[p + 2][q] = t[2], x[p + 3][q] = t[3];
            }
            if constexpr (F % 4 == 2) {  // whole tiles only (no EDGE)
                const auto t = gemm_f32_buffer_load_x2(rs, voff[0] + 4 * (F - 2), q * ld * 4, 0);
                x[F - 2][q] = t[0], x[F - 1][q] = t[1];
            }
        } else {
            const int o = kc && c * 16 >= klim ? kOut : voff[q];
            const floatx4 t = gemm_f32_buffer_load_x4(rs, o, 0, 0);
            x[q][0] = t[0], x[q][1] = t[1], x[q][2] = t[2], x[q][3] = t[3];
        }
    }
    template <bool KCHK>
    __device__ __forceinline__ void load(float (&x)[F][4], int c) const {
#pragma unroll
        for (int q = 0; q < kPieces; ++q) load_piece<KCHK>(x, c, q);
    }
};

// The 4 FM FN instructions of a chunk (sets xa, xb; s, then f, then j), then
// chunk c's loads into the same sets, each piece issued right after the last
// instruction that reads the registers it overwrites.
template <bool KCHK, int FM, int FN, class OA, class OB>
__device__ __forceinline__ void mma_reload(floatx4 (&acc)[FM][FN], float (&xa)[FM][4], float (&xb)[FN][4],
                                           const OA &la, const OB &lb, int c) {
    constexpr bool rowA = !OA::kKMajor, rowB = !OB::kKMajor;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[f][s], xb[j][s], acc[f][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!rowA) la.template load_piece<KCHK>(xa, c, s);
        if constexpr (!rowB) lb.template load_piece<KCHK>(xb, c, s);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int f = 0; f < FM; ++f) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[f][3], xb[j][3], acc[f][j], 0, 0, 0);
        if constexpr (rowA) {
            __builtin_amdgcn_sched_barrier(0);
            la.template load_piece<KCHK>(xa, c, f);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (!rowA) la.template load_piece<KCHK>(xa, c, 3);
    if constexpr (rowB) {
#pragma unroll
        for (int j = 0; j < FN; ++j) lb.template load_piece<KCHK>(xb, c, j);
    } else {
        lb.template load_piece<KCHK>(xb, c, 3);
    }
}

// EDGE: 0 = whole tiles and whole chunks (no checks), 1 = clamped loop and a
// zero-filled tail, 2 = every load checked (an extent below F - 1).
// OCC: wavefronts per SIMD at most (one workgroup per CU with OCC = 1: two
// 64 x 64 tiles that share a CU thrash its L1 and ran at half the rate).
// ET: the tail's loads go out before the loop, into registers of their own.
// TA / TB: op(A) = A^T (A stored K x M) / op(B) = B^T (B stored N x K).
template <int BM, int BN, int WM, int WN, int KG, int D, int OCC, bool ET, bool TA, bool TB, int EDGE>
__global__ __launch_bounds__(64 * WM * WN * KG) __attribute__((amdgpu_waves_per_eu(1, OCC)))
void gemm_mfma_regs_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n, int group_m, BatchArgs bt) {
    constexpr int NWG = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int CK = 16;  // k per chunk: four 16x16x4 instructions per block
    static_assert(WTM % 16 == 0 && (FN == 1 || FN == 2 || FN % 4 == 0), "16 x 16 blocks");
    static_assert(D >= 2, "at least two chunks in flight");
    constexpr int RP = KG > 1 ? regs_pass_rows(FM, FN, KG, NWG) : 1;
    static_assert(KG == 1 || RP > 0, "LDS room for the k-group sum");
    constexpr int RED = KG > 1 ? KG * NWG * RP * 64 * FN : 1;  // floats
    __shared__ __align__(16) float red[RED];

    int tm, tn;
    const int tile = batch_select(xcd_remap(blockIdx.x, tiles_m * tiles_n * bt.count),
                                  tiles_m * tiles_n, bt, A, B, C, K);
    grouped_tile(tile, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave / NWG, wg = wave % NWG;
    const int wm = wg / WN, wn = wg % WN;
    const int g = lane / 16, i = lane % 16;

    // A's blocks: rows 16 f + i of the slice (as stored) or FM i + f
    // (transposed, k-major); B's blocks: columns FN i + j either way.
    RegOperand<TA, FM, TA> opa;
    RegOperand<!TB, FN, true> opb;
    const int arow0 = m0 + wm * WTM, bcol = n0 + wn * WTN + FN * i;
    opa.init(A, lda, M, arow0, g, i, EDGE != 0);
    opb.init(B, ldb, N, n0 + wn * WTN, g, i, EDGE != 0);

    // Chunks of the loop (clamped addresses) and the tail chunk, if any.
    const int nloop = EDGE == 0 ? K / CK : EDGE == 1 ? (K - 1) / CK : 0;
    const int nchunks = EDGE == 0 ? nloop : (K + CK - 1) / CK;  // with the tail (or all, checked)
    // this group's chunks of the loop: kg, kg + KG, ...
    const int ng = nloop > kg ? (nloop - kg + KG - 1) / KG : 0;

    float ra[D][FM][4];
    float rb[D][FN][4];
    auto load = [&](float (&xa)[FM][4], float (&xb)[FN][4], int c) {
        opa.load(xa, c);
        opb.load(xb, c);
    };
    auto load_checked = [&](float (&xa)[FM][4], float (&xb)[FN][4], int c) {
        opa.load_checked(xa, c, g, K);
        opb.load_checked(xb, c, g, K);
    };

    floatx4 acc[FM][FN];
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[f][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // instructions s0, s0 + SS, ... of a chunk
    auto mma = [&](const float (&xa)[FM][4], const float (&xb)[FN][4], int s0 = 0, int ss = 1) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < s0 || (s - s0) % ss) continue;
#pragma unroll
            for (int f = 0; f < FM; ++f)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[f][s], xb[j][s], acc[f][j], 0, 0, 0);
        }
    };

    // The tail chunk (the one that holds the last k) is shared by the
    // groups: instruction s of it goes to group s mod KG.
    constexpr int TS = KG < 4 ? KG : 4;  // groups with a share of the tail
    const bool tail_mine = EDGE == 1 && nchunks > nloop && kg < TS;
    float ta[ET ? FM : 1][4];
    float tb[ET ? FN : 1][4];
    if constexpr (EDGE == 1 && ET) {
        if (tail_mine) load_checked(ta, tb, nloop);
    }

    if constexpr (EDGE == 2) {
        // every chunk checked (shapes too narrow for the clamped loads)
        for (int c = kg; c < nchunks; c += KG) {
            load_checked(ra[0], rb[0], c);
            mma(ra[0], rb[0]);
        }
    } else if (ng > 0) {
        // Set u holds the group's chunk t with t mod D = u; after the
        // instructions of chunk t, the same set loads chunk t + D (the last
        // chunk again past the end: in bounds, never used).
#pragma unroll
        for (int u = 0; u < D; ++u) load(ra[u], rb[u], kg + KG * min(u, ng - 1));
        int t = 0;
        for (; t + D <= ng; t += D) {
#pragma unroll
            for (int u = 0; u < D; ++u) {
                mma(ra[u], rb[u]);
                __builtin_amdgcn_sched_barrier(0);
                load(ra[u], rb[u], kg + KG * min(t + u + D, ng - 1));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int u = 0; u < D - 1; ++u)
            if (t + u < ng) mma(ra[u], rb[u]);
    }
    if constexpr (EDGE == 1) {
        if (tail_mine) {
            if constexpr (ET) {
                mma(ta, tb, kg, TS);
            } else {
                load_checked(ra[0], rb[0], nloop);
                mma(ra[0], rb[0], kg, TS);
            }
        }
    }

    // Register r of block (f, j): row 16 f + 4 g + r of the slice (A
    // transposed: FM (4 g + r) + f), column FN i + j.  With k-groups every wavefront leaves its partial slice in
    // LDS, RP rows (f, r) per pass, and the KG wavefronts that share a slice
    // each add up a KG-th of the pass's rows over the groups in group order
    // (a fixed order) and store them.
    const bool vec_c = (EDGE == 0 || (m0 + BM <= M && n0 + BN <= N)) &&
                       ((reinterpret_cast<uintptr_t>(C) | static_cast<uintptr_t>(ldc * 4)) &
                        (4 * (FN < 4 ? FN : 4) - 1)) == 0;
    auto store_row = [&](int fr, const float (&v)[FN]) {
        const int f = fr / 4, r = fr % 4;
        const int gm = arow0 + (TA ? FM * (4 * g + r) + f : 16 * f + 4 * g + r);
        float *row = C + static_cast<int64_t>(gm) * ldc + bcol;
        if (vec_c) {
            store_run<FN>(row, v);
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j)
                if (gm < M && bcol + j < N) row[j] = v[j];
        }
    };
    if constexpr (KG > 1) {
        // red[group][wave of group][row of the pass]: a lane's FN values as
        // FN / 4 pieces of 4 floats, piece p of all 64 lanes contiguous
        // (16-byte lane stride, no bank conflicts); FN < 4: [lane][j]
        auto part = [&](int h, int q, int p) {
            const int slot = (h * NWG + wg) * RP + q;
            return FN >= 4 ? red + ((slot * (FN / 4) + p) * 64 + lane) * 4 : red + slot * 64 * FN + lane * FN;
        };
#pragma unroll
        for (int pass = 0; pass < FM * 4 / RP; ++pass) {
            if (pass > 0) __syncthreads();  // the previous pass's reads are done
#pragma unroll
            for (int q = 0; q < RP; ++q) {
                const int fr = pass * RP + q;
                float v[FN];
#pragma unroll
                for (int j = 0; j < FN; ++j) v[j] = acc[fr / 4][j][fr % 4];
                if constexpr (FN >= 4) {
#pragma unroll
                    for (int p = 0; p < FN; p += 4)
                        *reinterpret_cast<floatx4 *>(part(kg, q, p / 4)) =
                            floatx4{v[p], v[p + 1], v[p + 2], v[p + 3]};
                } else {
                    store_run<FN>(part(kg, q, 0), v);
                }
            }
            __syncthreads();
#pragma unroll
            for (int qq = 0; qq < RP / KG; ++qq) {
                const int q = kg + qq * KG;
                float v[FN];
#pragma unroll
                for (int h = 0; h < KG; ++h) {
                    float x[FN];
                    if constexpr (FN >= 4) {
#pragma unroll
                        for (int p = 0; p < FN; p += 4) {
                            const floatx4 t4 = *reinterpret_cast<const floatx4 *>(part(h, q, p / 4));
                            x[p] = t4[0], x[p + 1] = t4[1], x[p + 2] = t4[2], x[p + 3] = t4[3];
                        }
                    } else if constexpr (FN == 2) {
                        const floatx2 t2 = *reinterpret_cast<const floatx2 *>(part(h, q, 0));
                        x[0] = t2[0], x[1] = t2[1];
                    } else {
                        x[0] = part(h, q, 0)[0];
                    }
#pragma unroll
                    for (int j = 0; j < FN; ++j) v[j] = h == 0 ? x[j] : v[j] + x[j];
                }
                store_row(pass * RP + q, v);
            }
        }
    } else {
#pragma unroll
        for (int fr = 0; fr < FM * 4; ++fr) {
            float v[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) v[j] = acc[fr / 4][j][fr % 4];
            store_row(fr, v);
        }
    }
}

// Barrier between the LDS writes and reads of the k-group sum that leaves
// global loads in flight: each wavefront waits for its own LDS accesses
// only (a __syncthreads would also wait for every outstanding global load,
// here the next tile's first chunks).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    // s_waitcnt: lgkmcnt 0; vmcnt 63 (bits 3:0 and 15:14) and expcnt 7 not waited on
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (3 << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Persistent form of the register-direct tile (whole tiles and K a multiple
// of 16 KG D; the EDGE form takes the rest): one workgroup per CU walks the
// tiles blockIdx.x +
// j gridDim.x (through the same XCD-aware, grouped order as the one-launch
// grid), and the last D chunks of a tile load the next tile's first D
// chunks into their register sets.  The next tile's loads are thus in
// flight during this tile's k-group sum and stores, and no workgroup start
// or first-load latency sits between two tiles of a CU.  Operands load as
// buffers (no vector address arithmetic), each piece of a set's next chunk
// right after the instructions that last read its registers (mma_reload).
// EDGE: edge tiles and K not a multiple of 16 KG D: rows past M or N and k
// past K load as zeros (BufOperand), each group runs K rounded up to whole
// rounds of D chunks, and stores past M or N are skipped.
template <int BM, int BN, int KG, int D, bool TA, bool TB, bool EDGE>
__global__ __launch_bounds__(64 * KG) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mfma_regs_persistent_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n, int group_m, BatchArgs bt) {
    constexpr int FM = BM / 16, FN = BN / 16;
    constexpr int CK = 16;
    static_assert(BM % 16 == 0 && (FN == 1 || FN == 2 || FN % 4 == 0), "16 x 16 blocks");
    static_assert(KG > 1 && D >= 2, "k-groups and chunks in flight");
    constexpr int RP = regs_pass_rows(FM, FN, KG, 1);
    static_assert(RP > 0, "LDS room for the k-group sum");
    __shared__ __align__(16) float red[KG * RP * 64 * FN];
    using OpA = BufOperand<TA, FM, TA, EDGE>;
    using OpB = BufOperand<!TB, FN, true, EDGE>;

    const int total = tiles_m * tiles_n * bt.count;
    const int G = static_cast<int>(gridDim.x);
    const int lane = threadIdx.x & 63;
    const int kg = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int g = lane / 16, i = lane % 16;
    // chunks of each group: kg, kg + KG, ... (with EDGE, K rounded up to
    // whole rounds of KG D chunks; the chunks past K load zeros)
    const int ng = EDGE ? (K + CK * KG * D - 1) / (CK * KG * D) * D : K / CK / KG;
    auto chunk_of = [&](int t) { return kg + KG * t; };

    // operands, C and origin of logical tile `logical`
    auto tile_at = [&](int logical, OpA &oa, OpB &ob, float *&c, int &m0, int &n0) {
        const float *a = A, *b = B;
        c = C;
        int k = K;
        const int t = batch_select(logical, tiles_m * tiles_n, bt, a, b, c, k);
        int tm, tn;
        grouped_tile(t, tiles_m, tiles_n, group_m, tm, tn);
        m0 = tm * BM, n0 = tn * BN;
        oa.init(a, lda, m0, g, i, M, K);
        ob.init(b, ldb, n0, g, i, N, K);
    };

    int logical = xcd_remap(static_cast<int>(blockIdx.x), G);
    if (logical >= total) return;
    OpA oa, oa_n;
    OpB ob, ob_n;
    float *c, *c_n;
    int m0, n0, m0_n, n0_n;
    tile_at(logical, oa, ob, c, m0, n0);

    float ra[D][FM][4];
    float rb[D][FN][4];
    floatx4 acc[FM][FN];
    // EDGE: the loads of a tile's first D chunks check k (a few per tile),
    // and so do those of the loop's rounds from t_chk on, the first round
    // that loads a chunk holding k past K; the rounds before do not
#pragma unroll
    for (int u = 0; u < D; ++u) {
        oa.template load<EDGE>(ra[u], chunk_of(u));
        ob.template load<EDGE>(rb[u], chunk_of(u));
    }
    int t_chk = ng;
    if constexpr (EDGE) {
        t_chk = 0;
        while (t_chk + D < ng && CK * chunk_of(t_chk + 2 * D - 1) + CK <= K) t_chk += D;
    }
    // slot of group h, pass row q: a lane's FN values as FN / 4 pieces of 4
    // floats, piece p of all 64 lanes contiguous (16-byte lane stride, no
    // bank conflicts); FN < 4: the lane's values adjacent
    auto part = [&](int h, int q, int p) {
        return FN >= 4 ? red + (((h * RP + q) * (FN / 4) + p) * 64 + lane) * 4
                       : red + (h * RP + q) * 64 * FN + lane * FN;
    };

    for (;;) {
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[f][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int next = logical + G;
        const bool has_next = next < total;
        auto round = [&](int t, auto kchk) {
#pragma unroll
            for (int u = 0; u < D; ++u) {
                __builtin_amdgcn_sched_barrier(0);
                mma_reload<decltype(kchk)::value>(acc, ra[u], rb[u], oa, ob, chunk_of(t + u + D));
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        int t = 0;
        for (; t + D < ng && t < t_chk; t += D) round(t, std::false_type{});
        if constexpr (EDGE)
            for (; t + D < ng; t += D) round(t, std::true_type{});
        // the last D chunks; their sets take the next tile's first D chunks
        // (the last tile reloads its own, in bounds and never used)
        if (has_next) {
            tile_at(next, oa_n, ob_n, c_n, m0_n, n0_n);
        } else {
            oa_n = oa, ob_n = ob, c_n = c, m0_n = m0, n0_n = n0;
        }
#pragma unroll
        for (int u = 0; u < D; ++u) {
            __builtin_amdgcn_sched_barrier(0);
            mma_reload<EDGE>(acc, ra[u], rb[u], oa_n, ob_n, chunk_of(u));
            __builtin_amdgcn_sched_barrier(0);
        }

        // the k-group sum in group order and the stores, as in the
        // one-launch kernel (register r of block (f, j): row 16 f + 4 g + r,
        // or FM (4 g + r) + f with A transposed; column FN i + j)
        const int bcol = n0 + FN * i;
        // vector stores where this product's C (its batch's, in a batch) and
        // ldc keep the runs aligned
        const bool vec_c = ((reinterpret_cast<uintptr_t>(c) | static_cast<uintptr_t>(ldc * 4)) &
                            (4 * (FN < 4 ? FN : 4) - 1)) == 0;
#pragma unroll
        for (int pass = 0; pass < FM * 4 / RP; ++pass) {
            lds_barrier();  // the previous reads of the LDS slots are done
#pragma unroll
            for (int q = 0; q < RP; ++q) {
                const int fr = pass * RP + q;
                float v[FN];
#pragma unroll
                for (int j = 0; j < FN; ++j) v[j] = acc[fr / 4][j][fr % 4];
                if constexpr (FN >= 4) {
#pragma unroll
                    for (int p = 0; p < FN; p += 4)
                        *reinterpret_cast<floatx4 *>(part(kg, q, p / 4)) =
                            floatx4{v[p], v[p + 1], v[p + 2], v[p + 3]};
                } else {
                    store_run<FN>(part(kg, q, 0), v);
                }
            }
            lds_barrier();
#pragma unroll
            for (int qq = 0; qq < RP / KG; ++qq) {
                const int q = kg + qq * KG;
                const int fr = pass * RP + q, f = fr / 4, r = fr % 4;
                float v[FN];
#pragma unroll
                for (int h = 0; h < KG; ++h) {
                    float x[FN];
                    if constexpr (FN >= 4) {
#pragma unroll
                        for (int p = 0; p < FN; p += 4) {
                            const floatx4 t4 = *reinterpret_cast<const floatx4 *>(part(h, q, p / 4));
                            x[p] = t4[0], x[p + 1] = t4[1], x[p + 2] = t4[2], x[p + 3] = t4[3];
                        }
                    } else if constexpr (FN == 2) {
                        const floatx2 t2 = *reinterpret_cast<const floatx2 *>(part(h, q, 0));
                        x[0] = t2[0], x[1] = t2[1];
                    } else {
                        x[0] = part(h, q, 0)[0];
                    }
#pragma unroll
                    for (int j = 0; j < FN; ++j) v[j] = h == 0 ? x[j] : v[j] + x[j];
                }
                const int gm = m0 + (TA ? FM * (4 * g + r) + f : 16 * f + 4 * g + r);
                float *row = c + static_cast<int64_t>(gm) * ldc + bcol;
                if (vec_c && (!EDGE || (m0 + BM <= M && n0 + BN <= N))) {
                    store_run<FN>(row, v);
                } else {
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        if (!EDGE || (gm < M && bcol + j < N)) row[j] = v[j];
                }
            }
        }
        if (!has_next) break;
        logical = next;
        oa = oa_n, ob = ob_n, c = c_n, m0 = m0_n, n0 = n0_n;
    }
}

// Launch of one configuration.
// WHOLE: compile the unchecked kernel for whole tiles and chunks (the
// 128 x 128 tiles spill registers in it and run the clamped one instead,
// whose last chunk is then a tail).
// PERSIST: the persistent kernel where the shape allows it (WM = WN = 1).
template <int BM, int BN, int WM, int WN, int KG, int D, int OCC, bool ET, bool WHOLE, int GROUP_M,
          bool PERSIST = false>
hipError_t launch_regs(const Problem &p, hipStream_t stream) {
    constexpr int NT = 64 * WM * WN * KG;
    constexpr int FM = BM / WM / 16, FN = BN / WN / 16;
    // A transposed (k-major) is loaded in runs of FM floats: FM of 1 or even
    // (configurations with other FM take A as stored only)
    constexpr bool kTransA = FM == 1 || FM % 2 == 0;
    if (p.ta && !kTransA) return hipErrorInvalidValue;
    const int tiles_m = ceil_div(p.M, BM), tiles_n = ceil_div(p.N, BN);
    const int64_t grid = static_cast<int64_t>(tiles_m) * tiles_n * p.batch;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool whole = p.M % BM == 0 && p.N % BN == 0 && p.K % 16 == 0 &&
                       (p.ksplit == 0 || p.ksplit % 16 == 0);
    // clamped k-major groups stay inside the operand when its rows are at
    // least one group less one long
    const bool clamp_ok = (!p.ta || p.M >= FM - 1) && (p.tb || p.N >= FN - 1);
    const int edge = whole && WHOLE ? 0 : clamp_ok ? 1 : 2;
    const dim3 gd(static_cast<unsigned>(grid)), bd(NT);
    if constexpr (PERSIST) {
        // one workgroup per CU walks the tiles: every tile the same K (split-K
        // slices of equal length run as a batch of products of that length),
        // a chunk's buffer offsets below 2^31 bytes, and whole tiles with K
        // whole rounds of D chunks per group, or else (EDGE form) K and the
        // rows of a k-major operand multiples of 4
        Problem q = p;
        if (p.ksplit > 0 && static_cast<int64_t>(p.batch) * p.ksplit == p.K) q.K = p.ksplit, q.ksplit = 0;
        const bool buf_ok = (q.ta ? 15 * q.lda + BM : (BM - 1) * q.lda + 16) < (int64_t{1} << 28) &&
                            (q.tb ? (BN - 1) * q.ldb + 16 : 15 * q.ldb + BN) < (int64_t{1} << 28);
        const bool whole_p = q.M % BM == 0 && q.N % BN == 0 && q.K % (16 * KG * D) == 0;
        const bool edge_p = q.K % 4 == 0 && (!q.ta || (q.M % 4 == 0 && FM % 4 == 0)) &&
                            (q.tb || (q.N % 4 == 0 && FN % 4 == 0));
        if (q.ksplit == 0 && buf_ok && q.K > 0 && (whole_p || edge_p)) {
            int dev = 0, cus = 0;
            hipError_t e = hipGetDevice(&dev);
            if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
            if (e != hipSuccess) return e;
            const unsigned wgs = static_cast<unsigned>(grid < cus ? grid : cus);
#define GEMM_REGS_P1(TA_, TB_, E)                                                                       \
    hipLaunchKernelGGL((gemm_mfma_regs_persistent_kernel<BM, BN, KG, D, TA_, TB_, E>), dim3(wgs), bd, 0, \
                       stream, q.M, q.N, q.K, q.A, q.lda, q.B, q.ldb, q.C, q.ldc, tiles_m, tiles_n,     \
                       GROUP_M, batch_of(q))
#define GEMM_REGS_P(TA_, TB_)                                                          \
    do {                                                                               \
        if (whole_p) GEMM_REGS_P1(TA_, TB_, false);                                    \
        else if constexpr ((!TA_ || FM % 4 == 0) && (TB_ || FN % 4 == 0))             \
            GEMM_REGS_P1(TA_, TB_, true);                                              \
    } while (0)
            if constexpr (kTransA) {
                if (p.ta && p.tb) GEMM_REGS_P(true, true);
                else if (p.ta) GEMM_REGS_P(true, false);
            }
            if (p.tb && !p.ta) GEMM_REGS_P(false, true);
            else if (!p.ta) GEMM_REGS_P(false, false);
#undef GEMM_REGS_P
#undef GEMM_REGS_P1
            return hipGetLastError();
        }
    }
#define GEMM_REGS(TA_, TB_, E)                                                                      \
    hipLaunchKernelGGL((gemm_mfma_regs_kernel<BM, BN, WM, WN, KG, D, OCC, ET, TA_, TB_, E>), gd, bd, \
                       0, stream, p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m,       \
                       tiles_n, GROUP_M, batch_of(p))
#define GEMM_REGS_E(TA_, TB_)                       \
    do {                                            \
        if (edge == 1) GEMM_REGS(TA_, TB_, 1);      \
        else if (edge == 2) GEMM_REGS(TA_, TB_, 2); \
        else if constexpr (WHOLE) GEMM_REGS(TA_, TB_, 0); \
    } while (0)
    if constexpr (kTransA) {
        if (p.ta && p.tb) GEMM_REGS_E(true, true);
        else if (p.ta) GEMM_REGS_E(true, false);
    }
    if (p.tb && !p.ta) GEMM_REGS_E(false, true);
    else if (!p.ta) GEMM_REGS_E(false, false);
#undef GEMM_REGS_E
#undef GEMM_REGS
    return hipGetLastError();
}

const ConfigEntry kRegsConfigs[] = {
    // operands straight from global memory into registers (mfmag): four
    // k-groups of one wavefront that each own the whole tile (no operand
    // loaded twice), D chunks in flight per wavefront, one wavefront per
    // SIMD.  (The K-step in the name is KG chunks of 16.)  Measured and not
    // kept: four wavefronts per group (w4x1, w2x2: each operand loaded by two
    // or four wavefronts; ragged 1000 x 1023 x 777 32 against 21 us), eight
    // groups of one wavefront (two per SIMD), 32 x 64 and 128 x 64 tiles,
    // D from 2 to 6 (within 2%), and loads spread between the MFMAs: into a
    // third register set (2 to 3% slower), into the set the previous chunk
    // freed (one chunk less lead: 0.5% slower at 128 x 128, 8% at 64 x 64),
    // or into the chunk's own set, each piece right after the last
    // instruction that reads its registers (1 to 10% slower with global
    // loads; with buffer loads, as the persistent tile runs them, the 64 x 64
    // tile gained nothing and the 128 x 128 one spilled registers).
    {"mfmag_64x64x64_w1x1_k4_d3", launch_regs<64, 64, 1, 1, 4, 3, 1, true, true, 8>, kCapTransposed},
    // 16 x 16: 256 workgroups at 256^3 (3.64 us median in a kernel trace
    // against 3.84 for the 16 x 16 LDS-staged tile; D 4 3.72, a 32 x 32
    // tile 4.64)
    {"mfmag_16x16x64_w1x1_k4_d2", launch_regs<16, 16, 1, 1, 4, 2, 1, true, true, 8>, kCapTransposed},
    // 128 x 128: 256 accumulator floats per lane
    {"mfmag_128x128x64_w1x1_k4_d2", launch_regs<128, 128, 1, 1, 4, 2, 1, true, false, 8>, kCapTransposed},
    // persistent where the shape allows (one workgroup per CU walks its
    // tiles; for the 64 x 64 tile it gained nothing, and a 64 x 128 one, D 2
    // or 4, ran within 1% of this tile from 2048^3 to 8192^3 and below the
    // library's two-launch plans where this tile's rounds quantise badly:
    // 4608^3 139.7 against 144.5, 5120^3 144.7 against 146.9 TFLOP/s)
    {"mfmag_128x128x64_w1x1_k4_d2_p", launch_regs<128, 128, 1, 1, 4, 2, 1, true, false, 8, true>, kCapTransposed},
    // 96 x 128: 768 tiles at 3072^3, three rounds of 256 (its edge form
    // takes A as stored; a transposed A runs whole tiles persistent, the
    // rest one launch per tile)
    {"mfmag_96x128x64_w1x1_k4_d2_p", launch_regs<96, 128, 1, 1, 4, 2, 1, true, false, 8, true>,
     kCapTransposed},
};

}  // namespace

const ConfigEntry *mfma_regs_configs(int *count) {
    *count = static_cast<int>(sizeof(kRegsConfigs) / sizeof(kRegsConfigs[0]));
    return kRegsConfigs;
}

}  // namespace gemm_f32_impl
