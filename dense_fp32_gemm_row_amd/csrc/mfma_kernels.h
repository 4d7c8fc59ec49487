// Stage 4: FP32 matrix cores (MFMA) with double-buffered LDS staging.
//
// Same blocking as the earlier stages -- a workgroup owns a BM x BN tile of
// C and walks K in steps of BK through LDS ("Tiled GEMM: Matrix
// Multiplication in CUDA", section 2) -- with three changes for CDNA4:
//
//  * The inner product runs on the FP32 matrix cores: v_mfma_f32_32x32x2_f32
//    adds a 32 x 2 slice of A times a 2 x 32 slice of B into a 32 x 32
//    accumulator block held in 16 registers per lane, v_mfma_f32_16x16x4_f32
//    a 16 x 4 slice times a 4 x 16 slice into a 16 x 16 block in 4
//    registers (the same rate; the instruction shape is a tuning axis).  Each
//    wavefront owns a (BM / WM) x (BN / WN) sub-tile, i.e. FM x FN
//    accumulator blocks: the register patch of "Tiling and Blocking for
//    Reuse" ("the next level: register blocking"), at wavefront granularity.
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
//    The pipelined kernel keeps direct global-to-LDS loads for them: with
//    16-byte-aligned rows, loads past M or N are clamped into the operand
//    (they only feed outputs that are never stored) and a partial last
//    K-step is staged through registers; without aligned rows, 4-byte
//    buffer loads return zero for every element outside the operand.  The
//    pipelined kernel's register staging clamps its loads the same way over
//    the whole K-steps and stages the K-step of the last k as a zero-filled
//    tail, so its K loop has no per-element checks either.
//
// This header holds two kernels: the first MFMA kernel (gemm_mfma_kernel,
// register staging, two LDS buffers) and the pipelined one
// (gemm_mfma_ring_kernel: a ring of two or three LDS buffers, fragment
// prefetch, optional direct global-to-LDS loads, XOR-swizzled A rows,
// interleaved B column blocks, transposed operands, k-groups that share
// each K-step between groups of wavefronts, and either instruction shape).
// csrc/mfma.hip and csrc/mfma16.hip list the compiled tile configurations.
//
// Operand layout.  For the 32x32x2 instruction lane l supplies A[l % 32][kk]
// and B[kk][l % 32] with kk = l / 32, and accumulator register r of lane l
// holds row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32.  For 16x16x4,
// lane l supplies A[l % 16][kk] and B[kk][l % 16] with kk = l / 16, and
// register r (0..3) holds row 4 * (l / 16) + r, column l % 16.  Within a
// chunk of 8 (16x16x4: 16) k values the kernel feeds instruction s
// (s = 0..3) with k = 4 * kk + s, a fixed permutation of the chunk applied
// to A and B alike, so lane l needs the 4 consecutive values
// A[m][4 * kk .. 4 * kk + 3]: one 16-byte LDS read per accumulator row block
// serves 4 instructions.  B, k-major in LDS, is read as single floats, 32
// (16) consecutive columns per lane group (or, with interleaved column
// blocks, as one 8- or 16-byte read per k).
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

#pragma once

#include <type_traits>

#include "gemm_internal.h"

namespace gemm_f32_impl {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// One FP32 matrix-core instruction on an MS x MS block: MS = 32 is
// v_mfma_f32_32x32x2_f32 (16 accumulator floats per lane), MS = 16 is
// v_mfma_f32_16x16x4_f32 (4 per lane).  Each lane supplies one value of A
// and one of B.
template <int MS>
struct MfmaShape;
template <>
struct MfmaShape<32> {
    using Acc = floatx16;
    static __device__ __forceinline__ Acc mma(float a, float b, Acc c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};
template <>
struct MfmaShape<16> {
    using Acc = floatx4;
    static __device__ __forceinline__ Acc mma(float a, float b, Acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

constexpr int kLdsBytes = 160 * 1024;  // LDS available to one workgroup on gfx950

// Four consecutive floats of one row starting at column `col`, zeros outside
// [0, limit) and for rows that do not exist (GUARD).  Four in-range floats are
// one 16-byte load: an aligned one when the row is 16-byte aligned (VEC),
// else four 4-byte loads that the compiler merges into one load, which
// global memory accepts at 4-byte alignment.
template <bool GUARD, bool VEC>
__device__ __forceinline__ float4 load_row4(const float *row_ptr, int col, int limit, bool row_ok) {
    if constexpr (!GUARD) {
        if constexpr (VEC) return *reinterpret_cast<const float4 *>(row_ptr + col);
        return make_float4(row_ptr[col], row_ptr[col + 1], row_ptr[col + 2], row_ptr[col + 3]);
    } else {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row_ok) {
            if (col + 3 < limit) {
                if constexpr (VEC) v = *reinterpret_cast<const float4 *>(row_ptr + col);
                else v = make_float4(row_ptr[col], row_ptr[col + 1], row_ptr[col + 2], row_ptr[col + 3]);
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
    int tiles_m, int tiles_n, int group_m, BatchArgs bt) {
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
    static_assert(2 * (BM * LDA_S + BK * LDB_S) * 4 <= kLdsBytes, "LDS budget of a workgroup");

    __shared__ __align__(16) float sA[2][BM * LDA_S];  // m-major, k contiguous
    __shared__ __align__(16) float sB[2][BK * LDB_S];  // k-major, n contiguous

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    int tm, tn;
    const int tile = batch_select(xcd_remap(blockIdx.x, tiles_m * tiles_n * bt.count),
                                  tiles_m * tiles_n, bt, A, B, C, K);
    grouped_tile(tile, tiles_m, tiles_n, group_m, tm, tn);
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

// Workgroup barrier for a loop whose direct global -> LDS loads run PENDING
// instructions ahead: the wavefront waits until at most its PENDING most
// recent vector-memory instructions are outstanding (they complete in
// order, so its older loads have landed in LDS) and its LDS reads are done,
// then meets the others.  __syncthreads() would wait for every outstanding
// load, because its workgroup fence does.  The empty asm statements keep
// the compiler from moving memory accesses across the wait (the count
// assumes the newest loads were issued before it) and LDS accesses across
// the barrier, as the fence did.
template <int PENDING>
__device__ __forceinline__ void barrier_after_older_loads() {
    static_assert(PENDING >= 0 && PENDING < 64, "vmcnt is 6 bits");
    asm volatile("" ::: "memory");
    // s_waitcnt: vmcnt in bits 3:0 and 15:14, lgkmcnt 0, expcnt (7) not waited on
    __builtin_amdgcn_s_waitcnt((PENDING & 15) | ((PENDING >> 4) << 14) | (7 << 4));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One operand of the pipelined kernel: the R x BK slice (R = BM rows of op(A)
// or BN columns of op(B)) that one K-step stages through LDS.
//
// Two storage flavours, chosen by how the operand lies in memory:
//  * row flavour (KMAJOR = false): element (r, k) at X[r * ld + k], k
//    contiguous -- A as stored, or B transposed.  LDS holds R rows of BK
//    floats; a lane's 4 values of one chunk (k = 4 kk .. 4 kk + 3, see the
//    operand layout above) are one 16-byte read.  The rows are padded by PAD
//    floats when PAD > 0, otherwise their 16-byte slots are XOR-swizzled.
//  * k-major flavour (KMAJOR = true): element (r, k) at X[k * ld + r], r
//    contiguous -- B as stored, or A transposed.  LDS holds BK rows of R
//    floats (+ PAD when PAD > 0); a lane reads its 4 values as 4 single
//    floats, 32 consecutive r per half wavefront.
// Register staging (with zero fill outside the matrix) and direct
// global -> LDS loads are provided for both.
// Whether an R x BK operand tile loaded by NW wavefronts can use 4-byte
// direct loads (see OperandTile): whole 256-byte chunks per wavefront, and a
// chunk stride of whole rows, which keeps a lane's column fixed (the k-major
// flavour) or cycles it through a few swizzled positions (the row flavour).
constexpr bool dw_tile_ok(int R, int BK, int NW, bool kmajor) {
    return (R * BK / 64) % NW == 0 && (kmajor ? (64 * NW) % R == 0 : (64 * NW) % BK == 0);
}
constexpr int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }

template <int R, int BK, int PAD, bool KMAJOR, int NT, int NW, bool GUARD, bool VEC, bool DIRECT,
          int IL = 1, int MS = 32>
struct OperandTile {
    static constexpr bool SWZ = !KMAJOR && PAD <= 0;
    static_assert(IL == 1 || (KMAJOR && (IL == 2 || IL == 4)), "interleave: k-major, 2 or 4 blocks");
    // Fragment geometry of the MFMA shape (MS x MS blocks): MS lanes along
    // the rows of a block, KK = 64 / MS lane groups along k, and a chunk of
    // CK = 4 KK values of k, of which each lane holds 4 consecutive ones.
    static_assert(MS == 32 || MS == 16, "32x32x2 or 16x16x4 instructions");
    static constexpr int KK = 64 / MS;
    static constexpr int CK = 4 * KK;
    static_assert(BK % CK == 0, "K-step of whole chunks");
    static constexpr int LD = KMAJOR ? R + (PAD > 0 ? PAD : 0) : BK + (SWZ ? 0 : PAD);  // row length
    static constexpr int SIZE = KMAJOR ? BK * LD : R * LD;               // floats per buffer
    static constexpr int L = (R * BK) / (4 * NT);                        // float4 slots per thread
    static constexpr int S = BK / 4;                                     // 16-byte slots per row
    static constexpr int LOG2S = S == 2 ? 1 : S == 4 ? 2 : S == 8 ? 3 : 4;
    static constexpr int CH = R * BK / 256;                              // 1 KiB chunks
    // Direct loads come in two kinds.  With 16-byte-aligned rows (VEC) one
    // global_load_lds_dwordx4 moves 1 KiB.  Without (DW) one 4-byte buffer
    // load into LDS moves 256 bytes, a float per lane, and a lane whose
    // element lies outside the operand (past K or past the R extent) gets an
    // offset outside the buffer's range, which the hardware's range check
    // turns into zero: zero fill with no registers, for edge tiles and a
    // partial last K-step alike.  A wavefront's successive 256-byte chunks
    // are NW chunks apart, DW_STEP whole rows: a lane keeps its column in the
    // k-major flavour, and in the row flavour its element's k column follows
    // the row's swizzle, which repeats every 32 rows (DW_P chunks).
    static constexpr bool DW = DIRECT && !VEC;
    static constexpr int CHW = R * BK / 64;                              // 256-byte chunks
    static constexpr int DW_STEP = KMAJOR ? 64 * NW / R : 64 * NW / BK;  // rows between them
    static constexpr bool DW_OK = dw_tile_ok(R, BK, NW, KMAJOR);
    static constexpr int J = DIRECT && !DW ? CH / NW : 1;
    static constexpr int JW = DW ? CHW / NW : 1;
    static constexpr int LOADS = DW ? JW : DIRECT ? J : 0;  // direct-load instructions per K-step
    static constexpr int DW_P = KMAJOR || !DW_OK ? 1 : 32 / gcd(DW_STEP, 32);
    static constexpr int DW_NC = DW_P < JW ? DW_P : JW;  // distinct k columns of a lane
    static_assert(L * 4 * NT == R * BK, "even tile split");
    static_assert(LD % 4 == 0, "16-byte aligned LDS rows");
    // Direct loads need unpadded LDS rows and 16-byte-aligned global rows.
    // With GUARD they serve tiles that overhang the operand's R extent (M or
    // N): the overhanging rows only feed outputs that are never stored, so
    // instead of zero fill their loads are clamped onto the last valid row
    // (row flavour) or 16-byte group (k-major flavour, which needs the R
    // extent to be a multiple of 4).  K must be whole K-steps.
    static_assert(!DIRECT || PAD <= 0, "direct loads: unpadded tiles");
    static_assert(!DIRECT || DW || CH % NW == 0, "whole chunks per wavefront");
    static_assert(!DW || DW_OK, "4-byte direct loads: chunk stride keeps swizzle and columns");

    // XOR swizzle of the row flavour: slot q of row m is stored at slot
    // q ^ g(m), g(m) = (r ^ (r >> log2 S)) mod S with r = m mod 32.  A
    // wavefront's 16-byte reads (32 consecutive rows of one 32-row block, one
    // slot) and its 16-byte stores (S lanes per row, 64 / S consecutive rows
    // inside one 32-row block) then hit disjoint banks, whether the LDS
    // serves 8 or 16 such accesses per cycle.  Depending on m mod 32 only,
    // g is the same for every 32-row block a lane reads.
    static __device__ __forceinline__ int swz(int m) {
        return ((m & 31) ^ ((m & 31) >> LOG2S)) & (S - 1);
    }

    const float *X;
    int64_t ld;
    int r0, rlim;
    int ro[L], co[L], st[L];  // tile coordinates and LDS offset of each slot
    // Register staging: one or two sets of the tile in flight, and the tail
    // step loaded early (two register sets).  Native vectors: with HIP's
    // float4 struct the copies became memcpys, and with the tail set live
    // across the loop the compiler kept them in scratch memory.
    floatx4 reg[2][L];
    floatx4 treg[L];
    const float *src[J];
    int dst[J];
    __amdgpu_buffer_rsrc_t rsrc;  // DW: the operand as a buffer
    int dw_off, dw_lim, dw_row;   // DW: lane's element offset (row flavour: of its row), k row
                                  // (k-major) and row of the first chunk (row flavour)
    int dw_kc[DW_NC];             // DW, row flavour: k column in chunks j = p mod DW_P

    __device__ __forceinline__ void init(const float *X_, int64_t ld_, int r0_, int rlim_, int tid,
                                         int wave, int lane) {
        X = X_, ld = ld_, r0 = r0_, rlim = rlim_;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int e = tid + i * NT;
            if constexpr (KMAJOR) {
                ro[i] = e / (R / 4);        // k row
                co[i] = (e % (R / 4)) * 4;  // r column
                st[i] = ro[i] * LD + co[i];
            } else {
                ro[i] = e / S;              // r row
                co[i] = (e % S) * 4;        // k column
                st[i] = ro[i] * LD + (SWZ ? ((co[i] / 4) ^ swz(ro[i])) * 4 : co[i]);
            }
        }
        if constexpr (DW) {
            // range up to 2^31 - 1 bytes: every valid offset is below it (the
            // launcher checks the operand's span), 0x80000000 is outside
            rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(X_), 0, 0x7fffffff,
                                                     0x00020000);
            const int f = wave * 64 + lane;  // float offset of the lane in its first chunk
            if constexpr (KMAJOR) {
                const int kr = f / R, col = f % R;
                dw_off = kr * static_cast<int>(ld_) + r0_ + col;
                dw_lim = r0_ + col < rlim_ ? kr : 0x40000000;  // k row; out-of-range column: never valid
            } else {
                // the lane's LDS position in chunk j is row m + j DW_STEP,
                // physical column f % BK, which holds the logical column
                // given by that row's swizzle
                const int m = f / BK;
#pragma unroll
                for (int p = 0; p < DW_NC; ++p)
                    dw_kc[p] = 4 * (((f % BK) / 4) ^ swz(m + p * DW_STEP)) + f % 4;
                dw_off = (r0_ + m) * static_cast<int>(ld_);
                dw_row = r0_ + m;
            }
        }
        if constexpr (DIRECT && !DW) {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int c = wave + j * NW;
                dst[j] = c * 256;
                if constexpr (KMAJOR) {
                    const int f = c * 256 + lane * 4;  // float offset in the k-major tile
                    int col = r0 + f % R;
                    if (GUARD && col > rlim - 4) col = rlim - 4;
                    src[j] = X + static_cast<int64_t>(f / R) * ld + col;
                } else {
                    const int m = c * (64 / S) + lane / S;  // tile row of this lane's slot
                    const int q = (lane % S) ^ swz(m);      // logical slot stored there
                    int row = r0 + m;
                    if (GUARD && row > rlim - 1) row = rlim - 1;
                    src[j] = X + static_cast<int64_t>(row) * ld + 4 * q;
                }
            }
        }
    }

    // Clamped register staging (edge tiles without per-element checks),
    // for K-steps that hold neither a k past K nor the operand's last k row
    // (k-major flavour): every load stays inside the operand's storage, and
    // the values of rows or columns past the R extent only feed outputs that
    // are never stored.  Row flavour: a row past the extent loads the last
    // row.  K-major flavour: a 4-column group that starts inside the extent
    // loads as it is, its columns past the extent coming from the row's
    // padding or the next row (a k row below the last one, so still inside
    // the storage when ld >= 4); a group wholly past the extent loads the
    // row's last group.  The slot's source is fixed for the tile; a K-step
    // adds k0 (row flavour) or k0 rows (k-major).
    const float *cp[L];
    __device__ __forceinline__ void init_clamp() {
#pragma unroll
        for (int i = 0; i < L; ++i) {
            if constexpr (KMAJOR) {
                const int last = (rlim - 1) & ~3;  // start of the last group inside the extent
                const int col = r0 + co[i] < rlim ? r0 + co[i] : last;
                cp[i] = X + static_cast<int64_t>(ro[i]) * ld + col;
            } else {
                const int row = r0 + ro[i] < rlim ? r0 + ro[i] : rlim - 1;
                cp[i] = X + static_cast<int64_t>(row) * ld + co[i];
            }
        }
    }
    template <int SET = 0>
    __device__ __forceinline__ void load_clamped(int k0) {
        const int64_t step = KMAJOR ? static_cast<int64_t>(k0) * ld : k0;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const float *q = cp[i] + step;
            if constexpr (VEC) reg[SET][i] = *reinterpret_cast<const floatx4 *>(q);
            else reg[SET][i] = floatx4{q[0], q[1], q[2], q[3]};
        }
    }

    // Register staging of the tile of K-step starting at k0 (G: with zero
    // fill outside the operand; the direct-load kernels use it for a
    // partial last K-step).
    template <int SET>
    __device__ __forceinline__ void set_reg(int i, float4 v) {
        const floatx4 x = {v.x, v.y, v.z, v.w};
        if constexpr (SET == 2) treg[i] = x;
        else reg[SET][i] = x;
    }
    // (V16 = false: four 4-byte loads that the compiler merges where all four
    // are in range, also for aligned rows)
    template <bool G = GUARD, int SET = 0, bool V16 = VEC>
    __device__ __forceinline__ void load(int k0, int K) {
#pragma unroll
        for (int i = 0; i < L; ++i) {
            if constexpr (KMAJOR) {
                const int gk = k0 + ro[i];
                const bool ok = !G || gk < K;
                const float *row = X + static_cast<int64_t>(ok ? gk : 0) * ld + r0;
                set_reg<SET>(i, load_row4<G, V16>(row, co[i], rlim - r0, ok));
            } else {
                const bool ok = !G || r0 + ro[i] < rlim;
                const float *row = X + static_cast<int64_t>(ok ? r0 + ro[i] : 0) * ld;
                set_reg<SET>(i, load_row4<G, V16>(row, k0 + co[i], K, ok));
            }
        }
    }
    template <int SET = 0>
    __device__ __forceinline__ void store(float *buf) const {
#pragma unroll
        for (int i = 0; i < L; ++i)
            *reinterpret_cast<floatx4 *>(&buf[st[i]]) = SET == 2 ? treg[i] : reg[SET & 1][i];
    }

    // Direct loads of the tile of K-step k0 into `buf`: one instruction moves
    // 64 x 16 bytes into 1 KiB of contiguous LDS, lane L's 16 bytes at offset
    // 16 L; each lane fetches the element that belongs at its slot (for the
    // row flavour, the inverse of the swizzle).
    __device__ __forceinline__ void load_direct(int k0, int K, float *buf) const {
        typedef const __attribute__((address_space(1))) void *gptr_t;
        typedef __attribute__((address_space(3))) void *lptr_t;
        if constexpr (DW) {
            const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
#pragma unroll
            for (int j = 0; j < JW; ++j) {
                int off;
                bool ok;
                if constexpr (KMAJOR) {  // chunk j holds k rows DW_STEP * j further on
                    off = dw_off + (k0 + j * DW_STEP) * static_cast<int>(ld);
                    ok = dw_lim + j * DW_STEP + k0 < K;
                } else {                 // ... rows DW_STEP * j further down
                    const int kc = dw_kc[j % DW_P];
                    off = dw_off + j * DW_STEP * static_cast<int>(ld) + kc + k0;
                    ok = dw_row + j * DW_STEP < rlim && kc + k0 < K;
                }
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (lptr_t)(&buf[(wave + j * NW) * 64]), 4,
                    ok ? off * 4 : static_cast<int>(0x80000000u), 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const float *g = KMAJOR ? src[j] + static_cast<int64_t>(k0) * ld : src[j] + k0;
                __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)(&buf[dst[j]]), 16, 0, 0);
            }
        }
    }

    // Per-lane part of the fragment reads of F blocks of MS rows starting at
    // row `rbase`, for lane lr of lane group g (lane = g MS + lr): an LDS
    // offset computed once, outside the K loop.  It is kept as one opaque
    // value so that the read addresses stay a short chain of offsets from
    // the LDS array (buffer, lane offset, chunk slot): the compiler's alias
    // scopes for the LDS arrays only reach that far, and without them it
    // cannot tell these reads from the direct loads of the other buffer and
    // waits for those loads before every K-step.
    // `kb`: first chunk of CK k that the wave reads (its k-group's share of
    // the K-step); chunk indices passed to read() count from there.
    // The swizzle of a row depends on the row mod 32: with 16-row blocks the
    // blocks at odd multiples of 16 rows past rbase use rg1.
    int rd, rg, rg1, rh;
    __device__ __forceinline__ void init_read(int rbase, int g, int lr, int kb = 0) {
        if constexpr (KMAJOR) {
            rd = 4 * g * LD + rbase + IL * lr + kb * CK * LD;
        } else {
            rd = (rbase + lr) * LD;
            rg = SWZ ? swz(rbase + lr) : 0;
            rg1 = SWZ ? swz(rbase + lr + 16) : 0;
            rh = g + KK * kb;  // slot KK (kb + kc) + g, before the swizzle
        }
        asm("" : "+v"(rd));
    }

    // The 4 values (k = kc CK + 4 g + s, s = 0..3) of F blocks of MS rows,
    // for the lane set up by init_read.  IL = 1: block f holds rows
    // MS f + lr of the wave's slice.  IL = F (k-major only): block f holds
    // rows F lr + f, so a lane's F values of one k are adjacent in LDS and
    // come in one vector read.

    template <int F>
    __device__ __forceinline__ void read(const float *buf, int kc, float (&v)[F][4]) const {
        if constexpr (KMAJOR && IL == 4) {
            static_assert(F == 4, "interleave width = blocks per wave");
            const float *p = buf + rd + kc * CK * LD;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float4 q = *reinterpret_cast<const float4 *>(p + s * LD);
                v[0][s] = q.x, v[1][s] = q.y, v[2][s] = q.z, v[3][s] = q.w;
            }
        } else if constexpr (KMAJOR && IL == 2) {
            static_assert(F == 2, "interleave width = blocks per wave");
            const float *p = buf + rd + kc * CK * LD;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float2 q = *reinterpret_cast<const float2 *>(p + s * LD);
                v[0][s] = q.x, v[1][s] = q.y;
            }
        } else if constexpr (KMAJOR) {
            const float *p = buf + rd + kc * CK * LD;
#pragma unroll
            for (int f = 0; f < F; ++f)
#pragma unroll
                for (int s = 0; s < 4; ++s) v[f][s] = p[s * LD + f * MS];
        } else {
            const int slot0 = SWZ ? (KK * kc + rh) ^ rg : KK * kc + rh;
            const int slot1 = SWZ ? (KK * kc + rh) ^ rg1 : KK * kc + rh;
            const float *p0 = buf + rd + slot0 * 4;
            const float *p1 = buf + rd + slot1 * 4;
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const float *p = (MS == 16 && (f & 1)) ? p1 : p0;
                const float4 q = *reinterpret_cast<const float4 *>(p + f * MS * LD);
                v[f][0] = q.x, v[f][1] = q.y, v[f][2] = q.z, v[f][3] = q.w;
            }
        }
    }

    // LDS read instructions per chunk for F blocks (pairs of k-major blocks
    // MS floats apart merge into one two-address read; interleaved blocks
    // are one vector read per k).
    template <int F>
    static constexpr int reads() { return KMAJOR ? (IL > 1 ? 4 : 4 * ((F + 1) / 2)) : F; }
};

// Pipelined kernel, with a ring of STAGES (2 or 3) LDS buffers.  Within a
// K-step the fragments of the next chunk of 8 k are read while the MFMAs of
// the current chunk run (two register sets, alternating).  With three
// buffers, in addition, the tile of K-step t + 1 is complete and published
// (by the barrier that ended step t - 1) while step t still runs, so each
// wavefront reads its first operand fragments of step t + 1 before the
// barrier that ends step t, and the matrix cores restart right after the
// barrier instead of waiting on LDS.
//
// Hazards, with three buffers and b(t) = t mod 3: step t writes tile t + 2 into
// b(t + 2) = b(t - 1), last read in step t - 1, i.e. before the barrier that
// ended step t - 1 (write after read); tile t + 2 is first read in step
// t + 1, after the barrier that ends step t (read after write).  Two buffers:
// see the barrier placement in the K loop.
//
// TA / TB: op(A) = A^T (A stored K x M) / op(B) = B^T (B stored N x K); a
// transposed operand swaps storage flavour (see OperandTile), nothing else
// changes.
//
// IL: when B's tile is k-major (B as stored), interleave the wave's column
// blocks: lane l32 of block j owns column FN l32 + j of the wave's columns
// instead of 32 j + l32.  A lane's B values of one k are then FN adjacent
// floats, one LDS read instead of FN / 2 two-address reads, and its
// outputs in one row are FN adjacent floats, one vector store.  Likewise
// for A's row blocks when A's tile is k-major (A transposed) and B's is
// too: row block i of lane l32 is row FM l32 + i.
//
// KG > 1: K-groups.  The workgroup holds KG groups of WM x WN wavefronts
// that all load each K-step's tiles together, but each group multiplies
// only its own BK / KG slice of the step (group g: chunks of 8 k
// g KC .. g KC + KC - 1), into accumulators for the whole tile.  The
// groups' partial tiles are then added in LDS, group 0 + group 1 + ...,
// a fixed order, and group 0 stores the sum.  For shapes with about one
// tile per CU this puts KG times more wavefronts on each SIMD to hide
// load and LDS latency, with no extra launch or workspace.
//
// One output tile of the pipelined kernel: the K loop and the epilogue for
// the tile at (m0, n0), with the LDS buffers of the workgroup.
template <int BM, int BN, int BK, int WM, int WN, int PADA, int PADB, int STAGES, bool DIRECT,
          bool GUARD, bool VEC, bool TA, bool TB, bool IL, int KG = 1, bool CL = false,
          int MS = 32, int RSETS = 1>
struct RingTile {
    // CL: register staging of an edge launch with clamped loads over the
    // whole K-steps and the partial last K-step as a zero-filled tail.
    static_assert(!CL || (GUARD && !DIRECT), "clamped loads: register staging with edges");
    // RSETS = 2: register staging with two register sets, so that the loads
    // of a K-step are issued two steps before their LDS store (two LDS
    // buffers): twice the time for them to land.
    static_assert(RSETS == 1 || (RSETS == 2 && STAGES == 2 && !DIRECT),
                  "two register sets: register staging with two LDS buffers");
    static constexpr bool TAIL = (DIRECT && VEC) || CL;  // a partial last K-step runs after the loop
    static constexpr int NWG = WM * WN;  // wavefronts per k-group
    static constexpr int NW = NWG * KG, NT = 64 * NW;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    // MS x MS accumulator blocks of the wave tile; a chunk is CK k (four
    // instructions), NREG accumulator floats per lane and block
    using Shape = MfmaShape<MS>;
    using Acc = typename Shape::Acc;
    static constexpr int KK = 64 / MS, CK = 4 * KK, NREG = MS * MS / 64;
    static constexpr int FM = WTM / MS, FN = WTN / MS;
    static constexpr int KC = BK / CK / KG;  // chunks per K-step and k-group
    // Interleave of A's row blocks: only when B's tile is k-major as well.
    // With A transposed and B transposed (TT) it issued a third fewer LDS
    // reads for the same LDS busy cycles, the waves waited longer to issue
    // them, and MFMA busy fell from 93.3% to 91.2% (TT 146.8 -> 142.8
    // TFLOP/s, same box); with B as stored (TN) it gains 1.3%.
    static constexpr int ILA = (IL && TA && !TB) ? FM : 1;
    using TileA = OperandTile<BM, BK, PADA, TA, NT, NW, GUARD, VEC, DIRECT, ILA, MS>;
    static constexpr int ILB = (IL && !TB) ? FN : 1;  // interleave of B's column blocks
    using TileB = OperandTile<BN, BK, PADB, !TB, NT, NW, GUARD, VEC, DIRECT, ILB, MS>;
    static constexpr int kReadsPerChunk = TileA::template reads<FM>() + TileB::template reads<FN>();
    static constexpr int kMfmaPerChunk = FM * FN * 4;
    static constexpr int kPairs = kReadsPerChunk < kMfmaPerChunk ? kReadsPerChunk : kMfmaPerChunk;
    static_assert(WTM % MS == 0 && WTN % MS == 0, "wave tile is whole MS x MS blocks");
    static_assert(BK % (2 * CK * KG) == 0, "an even number of chunks per K-step and k-group");
    static_assert(NT <= 1024, "at most 16 wavefronts per workgroup");
    static_assert(STAGES == 2 || STAGES == 3 || (STAGES == 4 && DIRECT),
                  "two or three LDS buffers, or four with direct loads");
    static_assert(STAGES * (TileA::SIZE + TileB::SIZE) * 4 <= kLdsBytes, "LDS budget of a workgroup");


    template <int SA, int SB>
    static __device__ __forceinline__ void run(int M, int N, int K, const float *__restrict__ A,
                                               int64_t lda, const float *__restrict__ B,
                                               int64_t ldb, float *__restrict__ C, int64_t ldc,
                                               int m0, int n0, float (&sA)[STAGES][SA],
                                               float (&sB)[STAGES][SB]) {
        static_assert(SA == TileA::SIZE && SB == TileB::SIZE, "LDS buffers of this tile shape");
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int kg = wave / NWG, wg = wave % NWG;  // k-group, wavefront within it
        const int wm = wg / WN, wn = wg % WN;

        TileA ta;
        TileB tb;
        ta.init(A, lda, m0, M, tid, wave, lane);
        tb.init(B, ldb, n0, N, tid, wave, lane);
        if constexpr (CL) {
            ta.init_clamp();
            tb.init_clamp();
        }
        auto load_step = [&](int k0, int buf) {
            if constexpr (DIRECT) {
                ta.load_direct(k0, K, sA[buf]);
                tb.load_direct(k0, K, sB[buf]);
            } else if constexpr (CL) {
                ta.load_clamped(k0);
                tb.load_clamped(k0);
            } else {
                ta.load(k0, K);
                tb.load(k0, K);
            }
        };
        auto store_step = [&](int buf) {
            if constexpr (!DIRECT) {
                ta.store(sA[buf]);
                tb.store(sB[buf]);
            }
        };
        // register staging into (from) register set SET_C::value
        auto load_set = [&](int k0, auto set_c) {
            constexpr int SET = decltype(set_c)::value;
            if constexpr (CL) {
                ta.template load_clamped<SET>(k0);
                tb.template load_clamped<SET>(k0);
            } else {
                ta.template load<GUARD, SET>(k0, K);
                tb.template load<GUARD, SET>(k0, K);
            }
        };
        auto store_set = [&](int buf, auto set_c) {
            constexpr int SET = decltype(set_c)::value;
            ta.template store<SET>(sA[buf]);
            tb.template store<SET>(sB[buf]);
        };
        (void)load_set, (void)store_set;

        const int half = lane / MS;  // lane group along k
        const int l32 = lane % MS;   // row (column) of the lane in its block
        ta.init_read(wm * WTM, half, l32, kg * KC);
        tb.init_read(wn * WTN, half, l32, kg * KC);

        // Two fragment register sets: operands of one chunk of 8 k.
        float fa[2][FM][4];
        float fb[2][FN][4];
        auto read_frag = [&](int set, int buf, int kc) {
            ta.template read<FM>(sA[buf], kc, fa[set]);
            tb.template read<FN>(sB[buf], kc, fb[set]);
        };

        Acc acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < NREG; ++r) acc[i][j][r] = 0.0f;

        auto mfma_chunk = [&](int set) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = Shape::mma(fa[set][i][s], fb[set][j][s], acc[i][j]);
        };

        // Direct loads move whole K-steps only; a partial last K-step is
        // the tail below.  (Spelled as the rounded-up count minus the tail:
        // with K / BK as the trip count the compiler recomputed the global
        // addresses with a 64-bit multiply every K-step instead of advancing
        // them, and the 16-wave kernels lost 11%.)
        // With clamped loads the K-step that holds the last k always goes to
        // the tail, whole or partial.
        const int nk = CL ? (K - 1) / BK : (K + BK - 1) / BK - (TAIL && (K % BK) ? 1 : 0);
        auto issue_pairs = [&] {
            // Issue order for the scheduler: the reads of the next chunk go
            // out one per MFMA at the start of this chunk, so their latency
            // hides behind the remaining MFMAs and the matrix pipe never
            // waits for a burst of reads.
#pragma unroll
            for (int r = 0; r < kPairs; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            }
            if constexpr (kReadsPerChunk > kPairs)
                __builtin_amdgcn_sched_group_barrier(0x100, kReadsPerChunk - kPairs, 0);
            if constexpr (kMfmaPerChunk > kPairs)
                __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerChunk - kPairs, 0);
        };
        // With two register sets, the tail's zero-filled loads (set 2) go out
        // before the loop: their latency is then off the critical path.  (As
        // 4-byte loads: the aligned 16-byte form, held across the loop, made
        // the compiler keep it in scratch memory.)
        constexpr bool EARLY_TAIL = RSETS == 2 && TAIL;
        if constexpr (EARLY_TAIL) {
            if (CL || K % BK) {
                ta.template load<true, 2, false>(nk * BK, K);
                tb.template load<true, 2, false>(nk * BK, K);
            }
        }
        if constexpr (RSETS == 2) {
            // Two register sets: step t reads LDS buffer t % 2.  At its top
            // it loads step t + 2 into register set t % 2 (stored to LDS at
            // the end of step t - 1), and before its barrier it stores set
            // (t + 1) % 2 (step t + 1, loaded at the top of step t - 1) into
            // buffer (t + 1) % 2 (last read in step t - 1).  The loop runs
            // steps in pairs, so buffer and set indices are constants.
            using S0 = std::integral_constant<int, 0>;
            using S1 = std::integral_constant<int, 1>;
            if (0 < nk) {
                load_set(0, S0{});
                store_set(0, S0{});
            }
            if (1 < nk) load_set(BK, S1{});
            __syncthreads();
            read_frag(0, 0, 0);
            // The loads are unconditional (the last two steps load the last
            // whole step again, in bounds, and their stores are never read):
            // behind a branch the compiler could not tell whether they had
            // been issued, and waited for them before the store of step t + 1.
            auto kstep = [&](int t, auto set_c) {
                constexpr int CUR = decltype(set_c)::value, NXT = 1 - CUR;
                load_set(min(t + 2, nk - 1) * BK, set_c);
                __builtin_amdgcn_sched_barrier(0);  // the loads go out first
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const int set = kc & 1;
                    if (kc == KC - 1) {
                        // stale but in-bounds in the last step
                        store_set(NXT, std::integral_constant<int, NXT>{});
                        __builtin_amdgcn_sched_barrier(0);
                        __syncthreads();
                        read_frag(set ^ 1, NXT, 0);
                    } else {
                        read_frag(set ^ 1, CUR, kc + 1);
                    }
                    mfma_chunk(set);
                    issue_pairs();
                }
            };
            // Whole pairs in the loop, an odd last step after it: with the
            // second step of a pair behind a branch, the compiler moved the
            // loads of set 0 into that branch, next to their store.
            int t = 0;
            for (; t + 1 < nk; t += 2) {
                kstep(t, S0{});
                kstep(t + 1, S1{});
            }
            if (t < nk) kstep(t, S0{});
        } else {
#pragma unroll
        for (int st = 0; st < STAGES - 1; ++st) {
            if (st < nk) {
                load_step(st * BK, st);
                store_step(st);
            }
        }
        __syncthreads();
        read_frag(0, 0, 0);

        int cur = 0;  // t mod STAGES
        for (int t = 0; t < nk; ++t) {
            const int nxt = cur == STAGES - 1 ? 0 : cur + 1;
            const int ahead = cur == 0 ? STAGES - 1 : cur - 1;  // (t + STAGES - 1) mod STAGES
            if (t + STAGES - 1 < nk) load_step((t + STAGES - 1) * BK, ahead);
            // Branch-free so that the reads stay ahead of the MFMAs they feed
            // (a branch here lets the compiler sink them back to their use).
            //
            // Three buffers, register staging: the last chunk reads ahead into
            // step t + 1 (tile t + 1 was published by the previous barrier); the
            // barrier ends the step.
            //
            // Two buffers, and three with direct loads: the barrier sits before
            // the last chunk.  By then the last chunk's fragments are in
            // registers (so every read of buffer `cur` is done: write after
            // read) and tile t + 1 has landed in buffer `nxt` (read after
            // write), so right after the barrier the first fragments of step
            // t + 1 are read while the last chunk's MFMAs run.  With three (four)
            // buffers the loads of tile t + 2 (and t + 3) stay in flight across
            // the barrier: each tile gets two (three) steps to land.
            //
            // In the last step the look-ahead read of buffer `nxt` is unused; it
            // stays inside the buffer, which nobody writes after the barrier.
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const int set = kc & 1;
                if constexpr (STAGES == 2 || DIRECT) {
                    if (kc == KC - 1) {
                        store_step(nxt);  // register staging: stale but in-bounds in the last step
                        // keep all of the previous chunk's MFMAs ahead of the
                        // barrier: they cover the latency of the reads it waits for
                        __builtin_amdgcn_sched_barrier(0);
                        constexpr int L = TileA::LOADS + TileB::LOADS;
                        if constexpr (STAGES == 2) {
                            __syncthreads();
                        } else if (STAGES == 4 && t + 3 < nk) {  // tiles t + 2, t + 3 in flight
                            barrier_after_older_loads<STAGES == 4 ? 2 * L : 0>();
                        } else if (t + 2 < nk) {                 // tile t + 2 in flight
                            barrier_after_older_loads<L>();
                        } else {
                            barrier_after_older_loads<0>();
                        }
                        read_frag(set ^ 1, nxt, 0);
                    } else {
                        read_frag(set ^ 1, cur, kc + 1);
                    }
                } else {
                    read_frag(set ^ 1, kc + 1 < KC ? cur : nxt, kc + 1 < KC ? kc + 1 : 0);
                }
                mfma_chunk(set);
                // Issue order for the scheduler: the reads of the next chunk go
                // out one per MFMA at the start of this chunk, so their latency
                // hides behind the remaining MFMAs and the matrix pipe never
                // waits for a burst of reads.
#pragma unroll
                for (int r = 0; r < kPairs; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                }
                if constexpr (kReadsPerChunk > kPairs)
                    __builtin_amdgcn_sched_group_barrier(0x100, kReadsPerChunk - kPairs, 0);
                if constexpr (kMfmaPerChunk > kPairs)
                    __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerChunk - kPairs, 0);
            }
            if constexpr (STAGES == 3 && !DIRECT) {
                if (t + 2 < nk) store_step(ahead);
                if (t + 1 < nk) __syncthreads();
            }
            cur = nxt;
        }
        }

        // Tail of the direct-load and clamped kernels: the partial last
        // K-step, staged through registers with zero fill past K (and past
        // the M / N edges), once all waves are done with the loop's buffers.
        // One exposed global-load latency per tile (none with two register
        // sets, which load it before the loop); its registers are not live in
        // the loop otherwise.  A wavefront whose share of the step lies
        // wholly past K skips it: it holds only zeros.
        if constexpr (TAIL) {
            if (CL || K % BK) {
                if constexpr (!EARLY_TAIL) {
                    ta.template load<true>(nk * BK, K);
                    tb.template load<true>(nk * BK, K);
                }
                constexpr int TS = EARLY_TAIL ? 2 : 0;
                __syncthreads();
                ta.template store<TS>(sA[0]);
                tb.template store<TS>(sB[0]);
                __syncthreads();
                // (one test per wavefront: a test per chunk made the compiler
                // keep the fragments in scratch memory)
                if (nk * BK + kg * KC * CK < K) {
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) {
                        read_frag(0, 0, kc);
                        mfma_chunk(0);
                    }
                }
            }
        }

        if constexpr (KG > 1) {
            // Sum of the k-groups' partial tiles, in group order, through the
            // LDS buffers (every wavefront is done with them after the first
            // barrier): a wavefront's partial tile is one slot of PER_WAVE
            // floats, one 256-byte row per register; slots fill the A buffers,
            // then the B buffers.  CAP groups per round write their slots and
            // group 0 adds them.
            constexpr int PER_WAVE = FM * FN * NREG * 64;
            constexpr int SLOTS_A = (STAGES * TileA::SIZE) / PER_WAVE;
            constexpr int SLOTS = SLOTS_A + (STAGES * TileB::SIZE) / PER_WAVE;
            constexpr int CAP = SLOTS / NWG;
            static_assert(CAP >= 1, "LDS room for one partial tile");
            auto slot = [&](int q) -> float * {
                return q < SLOTS_A ? &sA[0][0] + q * PER_WAVE : &sB[0][0] + (q - SLOTS_A) * PER_WAVE;
            };
#pragma unroll
            for (int g0 = 1; g0 < KG; g0 += CAP) {
                __syncthreads();
                if (kg >= g0 && kg < g0 + CAP) {
                    float *p = slot((kg - g0) * NWG + wg) + lane;
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
#pragma unroll
                            for (int r = 0; r < NREG; ++r) p[((i * FN + j) * NREG + r) * 64] = acc[i][j][r];
                }
                __syncthreads();
                if (kg == 0) {
#pragma unroll
                    for (int g = 0; g < CAP && g0 + g < KG; ++g) {
                        const float *p = slot(g * NWG + wg) + lane;
#pragma unroll
                        for (int i = 0; i < FM; ++i)
#pragma unroll
                            for (int j = 0; j < FN; ++j)
#pragma unroll
                                for (int r = 0; r < NREG; ++r)
                                    acc[i][j][r] += p[((i * FN + j) * NREG + r) * 64];
                    }
                }
            }
            if (kg != 0) return;
        }

        // accumulator register r of lane l: row 4 KK (r / 4) + 4 (l / MS) + r % 4,
        // column l % MS of its block (32x32x2: 8 (r / 4) + 4 (l / 32) + r % 4;
        // 16x16x4: 4 (l / 16) + r); with interleaved row blocks (ILA) row rho
        // of block i is row ILA * rho + i of the wave, else MS i + rho
        const int wrow0 = m0 + wm * WTM;
        auto row_of = [&](int i, int r) {
            const int rho = 4 * KK * (r / 4) + 4 * half + r % 4;
            return wrow0 + (ILA > 1 ? ILA * rho + i : MS * i + rho);
        };
        if constexpr (ILB > 1) {
            // column block j of lane l32 is column ILB * l32 + j of the wave
            const int gn = n0 + wn * WTN + ILB * l32;
            const bool vec_c = (!GUARD || (m0 + BM <= M && n0 + BN <= N)) &&
                               ((reinterpret_cast<uintptr_t>(C) | static_cast<uintptr_t>(ldc * 4)) &
                                (4 * ILB - 1)) == 0;
            if (vec_c) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int r = 0; r < NREG; ++r) {
                        float *row = C + static_cast<int64_t>(row_of(i, r)) * ldc + gn;
                        if constexpr (ILB == 4)
                            *reinterpret_cast<float4 *>(row) =
                                make_float4(acc[i][0][r], acc[i][1][r], acc[i][2][r], acc[i][3][r]);
                        else
                            *reinterpret_cast<float2 *>(row) = make_float2(acc[i][0][r], acc[i][1][r]);
                    }
            } else {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int r = 0; r < NREG; ++r) {
                        const int gm = row_of(i, r);
                        float *row = C + static_cast<int64_t>(gm) * ldc + gn;
#pragma unroll
                        for (int j = 0; j < ILB; ++j)
                            if (!GUARD || (gm < M && gn + j < N)) row[j] = acc[i][j][r];
                    }
            }
        } else {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int gn = n0 + wn * WTN + j * MS + l32;
#pragma unroll
                    for (int r = 0; r < NREG; ++r) {
                        const int gm = row_of(i, r);
                        if (!GUARD || (gm < M && gn < N))
                            C[static_cast<int64_t>(gm) * ldc + gn] = acc[i][j][r];
                    }
                }
            }
        }
    }
};

template <int BM, int BN, int BK, int WM, int WN, int PADA, int PADB, int STAGES, bool DIRECT,
          bool GUARD, bool VEC, bool TA, bool TB, bool IL, int KG, bool CL, int MS, int RSETS>
__global__ __launch_bounds__(64 * WM * WN * KG) void gemm_mfma_ring_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n, int group_m, BatchArgs bt) {
    // DIRECT and GUARD together: direct loads clamped at the M and N edges
    // (see OperandTile) and guarded stores; K is whole K-steps.
    using Full = RingTile<BM, BN, BK, WM, WN, PADA, PADB, STAGES, DIRECT, GUARD, VEC, TA, TB, IL, KG,
                          CL, MS, RSETS>;

    __shared__ __align__(16) float sA[STAGES][Full::TileA::SIZE];
    __shared__ __align__(16) float sB[STAGES][Full::TileB::SIZE];

    int tm, tn;
    const int tile = batch_select(xcd_remap(blockIdx.x, tiles_m * tiles_n * bt.count),
                                  tiles_m * tiles_n, bt, A, B, C, K);
    grouped_tile(tile, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    Full::run(M, N, K, A, lda, B, ldb, C, ldc, m0, n0, sA, sB);
}

// PIPE = 0: the first kernel; PIPE = 2, 3 or 4: the pipelined kernel with
// that many LDS buffers (four for direct loads only: where the shape needs
// register staging, that kernel runs with three).  DIRECT: direct global -> LDS loads where the shape
// allows (full tiles, 16-byte-aligned rows), register staging otherwise.
// TRANS: also compiled for transposed operands (pipelined kernel only).
// IL: interleaved column blocks for B as stored (pipelined kernel only).
// KG: k-groups of WM x WN wavefronts (pipelined kernel only).
// MS: 32 (v_mfma_f32_32x32x2_f32) or 16 (v_mfma_f32_16x16x4_f32) blocks
// (16: pipelined kernel only).
// RSETS: 2 for two register sets in the register-staged kernels of a
// two-buffer configuration (RingTile); direct loads are unaffected.
template <int BM, int BN, int BK, int WM, int WN, int PADA, int PADB, int GROUP_M, int PIPE,
          bool DIRECT = false, bool TRANS = false, bool IL = false, int KG = 1, int MS = 32,
          int RSETS = 1>
hipError_t launch_mfma(const Problem &p, hipStream_t stream) {
    static_assert(!TRANS || PIPE > 0, "transposed operands need the pipelined kernel");
    static_assert(!IL || PIPE > 0, "interleaved blocks need the pipelined kernel");
    static_assert(KG == 1 || PIPE > 0, "k-groups need the pipelined kernel");
    static_assert(MS == 32 || PIPE > 0, "16 x 16 blocks need the pipelined kernel");
    static_assert(RSETS == 1 || PIPE == 2, "two register sets: two LDS buffers");
    constexpr int NT = 64 * WM * WN * KG;
    if ((p.ta || p.tb) && !TRANS) return hipErrorNotSupported;
    const int tiles_m = ceil_div(p.M, BM), tiles_n = ceil_div(p.N, BN);
    const int64_t grid = static_cast<int64_t>(tiles_m) * tiles_n * p.batch;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool vec = rows_aligned16(p.A, p.lda, p.sa) && rows_aligned16(p.B, p.ldb, p.sb);
    const bool edge_mn = (p.M % BM) || (p.N % BN);
    // Split-K products run over K slices of p.ksplit (the last one shorter):
    // every slice must be whole K-steps for the kernels without a K check.
    const bool edge_k = (p.K % BK) != 0 || (p.ksplit > 0 && (p.ksplit % BK) != 0);
    const dim3 g(static_cast<unsigned>(grid)), b(NT);
#define GEMM_RING(D, G, V, TA, TB, CL_)                                                        \
    hipLaunchKernelGGL(                                                                         \
        (gemm_mfma_ring_kernel<BM, BN, BK, WM, WN, PADA, PADB, ((D) || PIPE < 4 ? PIPE : 3), D, G, \
                               V, TA, TB, IL, KG, CL_, MS, ((D) ? 1 : RSETS)>),                      \
        g, b, 0,                                                                                \
        stream, p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n, GROUP_M,   \
        batch_of(p))
#define GEMM_RING_T(D, G, V, CL_)                                                               \
    do {                                                                                        \
        if constexpr (TRANS) {                                                                  \
            if (p.ta && p.tb) GEMM_RING(D, G, V, true, true, CL_);                              \
            else if (p.ta) GEMM_RING(D, G, V, true, false, CL_);                                \
            else if (p.tb) GEMM_RING(D, G, V, false, true, CL_);                                \
            else GEMM_RING(D, G, V, false, false, CL_);                                         \
        } else {                                                                                \
            GEMM_RING(D, G, V, false, false, CL_);                                              \
        }                                                                                       \
    } while (0)
#define GEMM_MFMA_LAUNCH(D, G, V, CL_)                                                          \
    do {                                                                                        \
        if constexpr (PIPE > 0)                                                                 \
            GEMM_RING_T(D, G, V, CL_);                                                          \
        else                                                                                    \
            hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, WM, WN, PADA, PADB, G, V>), g, b, 0, \
                               stream, p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc,       \
                               tiles_m, tiles_n, GROUP_M, batch_of(p));                         \
    } while (0)
    // Edge tiles of 16-byte-aligned rows clamp their direct loads by whole
    // 16-byte groups, which needs the k-major operands' row length (M for A
    // transposed, N for B as stored) to be a multiple of 4.
    const bool clamp_ok = !edge_mn || ((!p.ta || p.M % 4 == 0) && (p.tb || p.N % 4 == 0));
    // Rows not 16-byte aligned, or edge tiles that cannot clamp: 4-byte
    // direct loads with range-checked zero fill, where the tile shape allows
    // it and every element offset (with a tile's overhang) stays below 2^29
    // floats, the buffers' 32-bit range.
    if constexpr (DIRECT && PIPE > 0) {
        constexpr int NW = WM * WN * KG;
        const int64_t a_rows = p.ta ? p.K : p.M, a_cols = p.ta ? p.M : p.K;
        const int64_t b_rows = p.tb ? p.N : p.K, b_cols = p.tb ? p.K : p.N;
        constexpr int64_t kSpan = int64_t{1} << 29;
        const bool spans_ok = (a_rows + 256) * p.lda + a_cols + 256 < kSpan &&
                              (b_rows + 256) * p.ldb + b_cols + 256 < kSpan;
        if ((!vec || !clamp_ok) && spans_ok) {
        // 4-byte loads issue R * BK / 64 instructions per operand and K-step;
        // with three or four buffers one or two K-steps of them stay in flight
        // at a barrier, which the 6-bit load counter must be able to express.
        constexpr int kDwLoads = (BM * BK / 64 + BN * BK / 64) / NW;
        constexpr bool kDwCountOk = (PIPE > 2 ? PIPE - 2 : 0) * kDwLoads < 64;
#define GEMM_DW(TA_, TB_)                                                                       \
    if constexpr ((TRANS || (!TA_ && !TB_)) && kDwCountOk && dw_tile_ok(BM, BK, NW, TA_) &&     \
                  dw_tile_ok(BN, BK, NW, !TB_)) {                                               \
        if (p.ta == TA_ && p.tb == TB_) {                                                       \
            GEMM_RING(true, true, false, TA_, TB_, false);                                             \
            return hipGetLastError();                                                           \
        }                                                                                       \
    }
            GEMM_DW(false, false)
            GEMM_DW(false, true)
            GEMM_DW(true, false)
            GEMM_DW(true, true)
#undef GEMM_DW
        }
    }
    // Direct-load configurations with aligned rows keep direct loads for
    // any shape: loads past M or N are clamped into the operands (GUARD:
    // guarded stores), and a partial last K-step is staged at the end of the
    // K loop.
    constexpr bool kDirectAny = DIRECT && PIPE > 0;
    if (!edge_mn && !edge_k) {
        if (vec) GEMM_MFMA_LAUNCH(DIRECT, false, true, false);
        else GEMM_MFMA_LAUNCH(false, false, false, false);
    } else if (kDirectAny && vec && clamp_ok) {
        if constexpr (kDirectAny) {
            if (edge_mn) GEMM_RING_T(true, true, true, false);
            else GEMM_RING_T(true, false, true, false);
        }
    } else {
        // Register staging with edges: clamped loads (no per-element checks
        // in the K loop) when every k-major operand's rows are at least 4
        // floats apart, so that a group's reads past its row stay inside
        // the operand.
        const bool clamp_regs = (p.tb || p.ldb >= 4) && (!p.ta || p.lda >= 4);
        if (clamp_regs) {
            if (vec) GEMM_MFMA_LAUNCH(false, true, true, true);
            else GEMM_MFMA_LAUNCH(false, true, false, true);
        } else {
            if (vec) GEMM_MFMA_LAUNCH(false, true, true, false);
            else GEMM_MFMA_LAUNCH(false, true, false, false);
        }
    }
#undef GEMM_MFMA_LAUNCH
#undef GEMM_RING_T
#undef GEMM_RING
    return hipGetLastError();
}

}  // namespace
}  // namespace gemm_f32_impl
