// C-ABI entry points of libgemm_f32.so (declared in include/gemm_f32.h).
//
// The host workflow of "Tiled GEMM: Matrix Multiplication in CUDA",
// section 6 (allocate, copy in, launch asynchronously, copy back, free) is
// split at the launch: the caller owns allocation, copies and
// synchronisation; this library validates the arguments, picks a kernel and
// enqueues it on the caller's stream.

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include <algorithm>
#include <mutex>

#include "../../include/gemm_f32.h"
#include "gemm_internal.h"
#include "tune_table.inc"

namespace gemm_f32_impl {
namespace {

thread_local char g_last_error[256] = "";

void clear_error() { g_last_error[0] = '\0'; }

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

__global__ __launch_bounds__(256) void zero_fill_kernel(float *__restrict__ C, int M, int N,
                                                        int64_t ldc, int batch, int64_t sc) {
    const int64_t per = static_cast<int64_t>(M) * N;
    const int64_t total = per * batch;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t b = e / per, r = e - b * per;
        const int64_t i = r / N, j = r - i * N;
        C[b * sc + i * ldc + j] = 0.0f;
    }
}

// Split-K reduction: C = W_0 + W_1 + ... + W_{S-1}, summed in that order for
// every element, so the result does not depend on scheduling.  W_s is a
// packed M x N slice (leading dimension N) `slice` floats after W_{s-1}.
template <bool VEC4>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ W,
                                                            int64_t slice, int S, int M, int N,
                                                            float *__restrict__ C, int64_t ldc) {
    constexpr int V = VEC4 ? 4 : 1;
    const int64_t per_row = N / V;
    const int64_t total = static_cast<int64_t>(M) * per_row;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t i = e / per_row, j = (e - i * per_row) * V;
        const float *w = W + i * N + j;
        if constexpr (VEC4) {
            float4 acc = *reinterpret_cast<const float4 *>(w);
            for (int s = 1; s < S; ++s) {
                const float4 v = *reinterpret_cast<const float4 *>(w + s * slice);
                acc.x += v.x, acc.y += v.y, acc.z += v.z, acc.w += v.w;
            }
            *reinterpret_cast<float4 *>(C + i * ldc + j) = acc;
        } else {
            float acc = w[0];
            for (int s = 1; s < S; ++s) acc += w[s * slice];
            C[i * ldc + j] = acc;
        }
    }
}

// Split geometry: `want` splits of K, the length rounded up to a multiple of
// 32; returns the split length and sets the number of splits actually used.
// A kernel whose K-step does not divide the length (BK = 64 or 128) runs its
// K-checked path on every slice.
int split_len(int64_t K, int64_t want, int64_t *used) {
    int64_t len = (K + want - 1) / want;
    len = ((len + 31) / 32) * 32;
    if (len < 32) len = 32;
    *used = (K + len - 1) / len;
    return static_cast<int>(len);
}

// Library choice of the number of K splits: enough 128 x 128 tiles (the
// persistent register-direct tile that takes slices of equal length) to give
// every CU one, with at least 1024 k per split.
int64_t auto_splits(int64_t M, int64_t N, int64_t K) {
    constexpr int64_t kCUs = 256;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    int64_t s = (kCUs + tiles - 1) / tiles;
    const int64_t by_k = K / 1024;
    if (s > by_k) s = by_k;
    return s < 1 ? 1 : s;
}

const ConfigEntry *configs_of(int variant, int *count) {
    switch (variant) {
        case GEMM_F32_VARIANT_NAIVE: return naive_configs(count);
        case GEMM_F32_VARIANT_LDS: return lds_configs(count);
        case GEMM_F32_VARIANT_REGBLOCK: return regblock_configs(count);
        case GEMM_F32_VARIANT_MFMA: return mfma_configs(count);
        default: *count = 0; return nullptr;
    }
}

int find_config(int variant, const char *name) {
    int n = 0;
    const ConfigEntry *c = configs_of(variant, &n);
    for (int i = 0; i < n; ++i)
        if (std::strcmp(c[i].name, name) == 0) return i;
    return -1;
}

// Byte range [lo, hi) spanned by a rows x cols row-major matrix.
struct Span {
    uintptr_t lo, hi;
};
Span span_of(const void *p, int64_t rows, int64_t cols, int64_t ld) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    if (rows == 0 || cols == 0) return {lo, lo};
    const uint64_t elems = static_cast<uint64_t>(rows - 1) * static_cast<uint64_t>(ld) +
                           static_cast<uint64_t>(cols);
    return {lo, lo + elems * sizeof(float)};
}
// ... and of `batch` such matrices `stride` floats apart.
Span span_of_batch(const void *p, int64_t batch, int64_t stride, int64_t rows, int64_t cols,
                   int64_t ld) {
    Span s = span_of(p, rows, cols, ld);
    if (s.lo != s.hi && batch > 1) s.hi += static_cast<uint64_t>(batch - 1) * stride * sizeof(float);
    return s;
}
bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

int validate_sizes(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                   bool ta = false, bool tb = false) {
    constexpr int64_t kMax = 0x7fffffff;
    if (M < 0 || N < 0 || K < 0) return fail(GEMM_F32_EINVAL, "negative size M=%lld N=%lld K=%lld",
                                             (long long)M, (long long)N, (long long)K);
    if (M > kMax || N > kMax || K > kMax)
        return fail(GEMM_F32_EINVAL, "size above 2^31-1 (M=%lld N=%lld K=%lld)", (long long)M,
                    (long long)N, (long long)K);
    // a stored row of A holds K floats (M when transposed), of B N (K)
    const int64_t a_row = ta ? M : K, b_row = tb ? K : N;
    if (lda < (a_row > 1 ? a_row : 1))
        return fail(GEMM_F32_EINVAL, "lda=%lld < max(1, %s=%lld)", (long long)lda, ta ? "M" : "K",
                    (long long)a_row);
    if (ldb < (b_row > 1 ? b_row : 1))
        return fail(GEMM_F32_EINVAL, "ldb=%lld < max(1, %s=%lld)", (long long)ldb, tb ? "K" : "N",
                    (long long)b_row);
    if (ldc < (N > 1 ? N : 1)) return fail(GEMM_F32_EINVAL, "ldc=%lld < max(1, N=%lld)", (long long)ldc, (long long)N);
    // Largest flat element index must stay addressable with 64-bit offsets.
    const int64_t kLdMax = (int64_t{1} << 62) / (kMax + 1);
    if (lda > kLdMax || ldb > kLdMax || ldc > kLdMax)
        return fail(GEMM_F32_EINVAL, "leading dimension above %lld", (long long)kLdMax);
    return GEMM_F32_OK;
}

// Largest element offset the batch strides may span (keeps every byte
// offset well inside 64 bits).
constexpr int64_t kSpanMax = int64_t{1} << 58;

int validate_batch(int64_t batch, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t sa,
                   int64_t ldb, int64_t sb, int64_t ldc, int64_t sc) {
    if (batch < 0) return fail(GEMM_F32_EINVAL, "negative batch %lld", (long long)batch);
    if (batch > 0x7fffffff) return fail(GEMM_F32_EINVAL, "batch above 2^31-1");
    if (sa < 0 || sb < 0 || sc < 0) return fail(GEMM_F32_EINVAL, "negative batch stride");
    if (batch > 1 && M > 0 && N > 0) {
        const int64_t c_span = (M - 1) * ldc + N;
        if (sc < c_span)
            return fail(GEMM_F32_EINVAL, "strideC=%lld < %lld: the products' C regions overlap",
                        (long long)sc, (long long)c_span);
    }
    const int64_t n = batch > 1 ? batch - 1 : 0;
    if ((sa && n > kSpanMax / sa) || (sb && n > kSpanMax / sb) || (sc && n > kSpanMax / sc))
        return fail(GEMM_F32_EINVAL, "batch x stride spans more than 2^58 floats");
    (void)K, (void)lda, (void)ldb;
    return GEMM_F32_OK;
}

int validate(bool ta, bool tb, int64_t batch, int64_t M, int64_t N, int64_t K, const float *A,
             int64_t lda, int64_t sa, const float *B, int64_t ldb, int64_t sb, const float *C,
             int64_t ldc, int64_t sc) {
    int rc = validate_sizes(M, N, K, lda, ldb, ldc, ta, tb);
    if (rc != GEMM_F32_OK) return rc;
    rc = validate_batch(batch, M, N, K, lda, sa, ldb, sb, ldc, sc);
    if (rc != GEMM_F32_OK) return rc;
    if (M == 0 || N == 0 || batch == 0) return GEMM_F32_OK;
    const bool need_a = M > 0 && K > 0, need_b = K > 0 && N > 0;
    if (C == nullptr) return fail(GEMM_F32_EINVAL, "C is NULL with M*N > 0");
    if (need_a && A == nullptr) return fail(GEMM_F32_EINVAL, "A is NULL with M*K > 0");
    if (need_b && B == nullptr) return fail(GEMM_F32_EINVAL, "B is NULL with K*N > 0");
    if (reinterpret_cast<uintptr_t>(C) % 4 || (need_a && reinterpret_cast<uintptr_t>(A) % 4) ||
        (need_b && reinterpret_cast<uintptr_t>(B) % 4))
        return fail(GEMM_F32_EINVAL, "pointer not 4-byte aligned");
    const Span scs = span_of_batch(C, batch, sc, M, N, ldc);
    const Span sas = ta ? span_of_batch(A, batch, sa, K, M, lda) : span_of_batch(A, batch, sa, M, K, lda);
    const Span sbs = tb ? span_of_batch(B, batch, sb, N, K, ldb) : span_of_batch(B, batch, sb, K, N, ldb);
    if (need_a && overlaps(scs, sas)) return fail(GEMM_F32_EINVAL, "C overlaps A");
    if (need_b && overlaps(scs, sbs)) return fail(GEMM_F32_EINVAL, "C overlaps B");
    return GEMM_F32_OK;
}

// The tile configuration gemm_f32 uses for a shape: an exact entry of the
// tuned table if there is one, else the cost model's choice.  The model
// ("Tiling and Blocking for Reuse", choosing the tile size: reuse against
// occupancy and tails, settled by measurement): a CU receives
// n = ceil(tiles / CUs) tiles of a candidate, and the candidate's measured
// per-CU rate for a share of min(n, nrates) tiles (the last level also
// stands for larger shares, whose tiles queue behind those that fit at
// once) gives the predicted time n * 2 * bm * bn * (K + k0) / rate, k0 being
// the tile's fixed cost (prologue, and stores of C that no other
// workgroup's math hides) in k; rows that are not 16-byte aligned scale the
// rate by the candidate's measured factor.  A
// batch multiplies the tiles.  Transposed operands consider only
// configurations that take them.

// Predicted microseconds of one candidate on a (batch of) M x N x K.
double model_us(const ModelCandidate &m, int64_t batch, int64_t M, int64_t N, int64_t K,
                bool aligned, bool trans) {
    const int64_t tiles = ((M + m.bm - 1) / m.bm) * ((N + m.bn - 1) / m.bn) * batch;
    const int64_t n = (tiles + kModelCUs - 1) / kModelCUs;
    const int level = static_cast<int>(n < m.nrates ? n : m.nrates);
    // a persistent candidate runs K in whole rounds of whole_k, and its edge
    // form (tiles past M or N, K past whole rounds) at its edge rate
    const bool edge = m.whole_k > 0 && (M % m.bm || N % m.bn || K % m.whole_k);
    if (m.whole_k > 0) K = (K + m.whole_k - 1) / m.whole_k * m.whole_k;
    const double rate = m.gflops_per_cu[level > 0 ? level - 1 : 0] * (aligned ? 1.0 : m.unaligned) *
                        (trans ? m.trans : 1.0) * (edge ? m.edge : 1.0);
    return static_cast<double>(n) * 2.0 * m.bm * m.bn * (static_cast<double>(K) + m.k0) /
           (rate * 1e3);
}

// Configuration ids of the model's candidates (-1: not compiled) and whether
// each takes transposed operands, resolved once.
constexpr int kModelSize = static_cast<int>(sizeof(kModel) / sizeof(kModel[0]));
struct ModelIds {
    int id[kModelSize];
    bool trans[kModelSize];
};
const ModelIds &model_ids() {
    static const ModelIds ids = [] {
        ModelIds r{};
        int count = 0;
        const ConfigEntry *cfgs = configs_of(GEMM_F32_VARIANT_MFMA, &count);
        for (int i = 0; i < kModelSize; ++i) {
            r.id[i] = find_config(GEMM_F32_VARIANT_MFMA, kModel[i].config);
            r.trans[i] = r.id[i] >= 0 && (cfgs[r.id[i]].caps & kCapTransposed);
        }
        return r;
    }();
    return ids;
}
// What a product asks of a candidate besides its shape: a transposed
// operand (the candidate must take them; A, B transposed), split-K slices.
constexpr unsigned kOpsTrans = 1u, kOpsTransA = 2u, kOpsSplitK = 4u, kOpsTransB = 8u;
unsigned ops_of(bool ta, bool tb) {
    return (ta || tb ? kOpsTrans : 0u) | (ta ? kOpsTransA : 0u) | (tb ? kOpsTransB : 0u);
}

// A candidate with whole_k > 0 (a persistent kernel) is rated only for the
// products it runs in that form: no split-K slices, and whole tiles with K a
// multiple of whole_k, or (its edge form) K and the row length of a k-major
// operand (M for A transposed, N for B as stored) multiples of 4, for tiles
// whose k-major loads come in groups of 4 (bm, bn multiples of 64).
bool usable(int i, unsigned ops, int64_t M, int64_t N, int64_t K) {
    const ModelIds &ids = model_ids();
    if (ids.id[i] < 0 || ((ops & kOpsTrans) && !ids.trans[i])) return false;
    const ModelCandidate &m = kModel[i];
    if (m.whole_k == 0) return true;
    if ((ops & kOpsSplitK) || K <= 0) return false;
    const bool whole = M % m.bm == 0 && N % m.bn == 0 && K % m.whole_k == 0;
    const bool edge = K % 4 == 0 && (!(ops & kOpsTransA) || (M % 4 == 0 && m.bm % 64 == 0)) &&
                      ((ops & kOpsTransB) || (N % 4 == 0 && m.bn % 64 == 0));
    return whole || edge;
}

// The model's fastest candidate; returns its predicted microseconds.
double best_candidate(int64_t batch, int64_t M, int64_t N, int64_t K, unsigned ops, bool aligned,
                      int *config) {
    double best_t = 0.0;
    *config = -1;
    for (int i = 0; i < kModelSize; ++i) {
        if (!usable(i, ops, M, N, K)) continue;
        const double t = model_us(kModel[i], batch, M, N, K, aligned, ops & kOpsTrans);
        if (*config < 0 || t < best_t) *config = model_ids().id[i], best_t = t;
    }
    if (*config < 0) *config = 0;
    return best_t;
}

bool exact_entry(int64_t M, int64_t N, int64_t K, int *variant, int *config) {
    for (const TuneEntry &e : kTuneTable) {
        if (e.M == M && e.N == N && e.K == K) {
            const int id = find_config(e.variant, e.config);
            if (id >= 0) {
                *variant = e.variant;
                *config = id;
                return true;
            }
        }
    }
    return false;
}

void select_config(int64_t batch, int64_t M, int64_t N, int64_t K, int *variant, int *config,
                   unsigned ops = 0, bool aligned = true) {
    if (batch == 1 && !(ops & (kOpsTrans | kOpsSplitK)) && exact_entry(M, N, K, variant, config))
        return;
    *variant = GEMM_F32_VARIANT_MFMA;
    best_candidate(batch, M, N, K, ops, aligned, config);
}

// How gemm_f32 runs one product, or every product of a strided batch alike:
// one launch, or two on complementary parts of C.  Wave quantisation ("Tiling and Blocking for Reuse", choosing the
// tile size: the tail of the last wave) can leave the last wave of large
// tiles mostly empty, where small tiles lose per-CU rate everywhere.  A
// split runs a first slab of C rows (or columns) with one candidate, sized
// to whole waves of its tiles, and the rest with the model's choice for the
// remaining shape: for each candidate and each number w of waves (up to
// kSplitWaves), the largest whole-tile slab with at most w * CUs tiles.  It
// is taken when the model predicts at least kSplitGain less time, after
// kLaunchUs for the second launch.  Products the model puts under
// kSplitMinUs are not searched: a split could save less there than the
// search costs on the host.
struct Plan {
    int parts;            // 1 or 2
    int axis;             // 0: split the rows of C, 1: its columns
    int64_t split;        // rows (columns) of the first part
    int variant[2], config[2];
};
constexpr double kLaunchUs = 5.0;
constexpr double kSplitGain = 0.02;
constexpr int64_t kSplitWaves = 16;
constexpr double kSplitMinUs = 100.0;

Plan search_plan(int64_t batch, int64_t M, int64_t N, int64_t K, unsigned ops, bool aligned) {
    Plan plan{1, 0, 0, {GEMM_F32_VARIANT_MFMA, 0}, {0, 0}};
    if (M <= 0 || N <= 0 || K <= 0 || batch <= 0) {  // nothing to split
        select_config(batch > 0 ? batch : 1, M, N, K, &plan.variant[0], &plan.config[0], ops,
                      aligned);
        return plan;
    }
    if (batch == 1 && !(ops & kOpsTrans) && exact_entry(M, N, K, &plan.variant[0], &plan.config[0]))
        return plan;
    const double t1 = best_candidate(batch, M, N, K, ops, aligned, &plan.config[0]);
    if (t1 < kSplitMinUs) return plan;
    double best_t = t1 * (1.0 - kSplitGain);
    for (int i = 0; i < kModelSize; ++i) {
        if (!usable(i, ops, 0, 0, 0)) continue;  // operand forms (the shape per part below)
        const ModelCandidate &m = kModel[i];
        const int id = model_ids().id[i];
        for (int axis = 0; axis < 2; ++axis) {
            const int64_t along = axis == 0 ? M : N, across = axis == 0 ? N : M;
            const int64_t tile = axis == 0 ? m.bm : m.bn, other = axis == 0 ? m.bn : m.bm;
            // tiles per row (column) of tiles, over the whole batch
            const int64_t lanes = (across + other - 1) / other * batch;
            for (int64_t w = 1; w <= kSplitWaves; ++w) {
                const int64_t first = (w * kModelCUs / lanes) * tile;
                if (first <= 0) continue;
                if (first >= along) break;
                const int64_t m1 = axis == 0 ? first : M, n1 = axis == 0 ? N : first;
                const int64_t m2 = axis == 0 ? M - first : M, n2 = axis == 0 ? N : N - first;
                if (!usable(i, ops, m1, n1, K)) continue;
                int c2 = -1;
                const double t = model_us(m, batch, m1, n1, K, aligned, ops & kOpsTrans) +
                                 best_candidate(batch, m2, n2, K, ops, aligned, &c2) + kLaunchUs;
                // one configuration in two launches only looks faster: each
                // launch would count at the one-tile-per-CU rate, but the
                // second still waits for the first and starts from cold
                if (c2 == id) continue;
                if (t < best_t) {
                    best_t = t;
                    plan = Plan{2, axis, first, {GEMM_F32_VARIANT_MFMA, GEMM_F32_VARIANT_MFMA},
                                {id, c2}};
                }
            }
        }
    }
    return plan;
}

// search_plan with the last result of the calling thread kept: a loop over
// one shape searches once.
Plan plan_product(int64_t batch, int64_t M, int64_t N, int64_t K, unsigned ops, bool aligned) {
    struct Key {
        int64_t batch, M, N, K;
        unsigned ops;
        bool aligned;
    };
    thread_local Key last{-1, -1, -1, -1, 0u, false};
    thread_local Plan last_plan{};
    if (batch == last.batch && M == last.M && N == last.N && K == last.K && ops == last.ops &&
        aligned == last.aligned)
        return last_plan;
    last_plan = search_plan(batch, M, N, K, ops, aligned);
    last = Key{batch, M, N, K, ops, aligned};
    return last_plan;
}

// Rows of A and B 16-byte aligned in every product.
bool operands_aligned(const float *A, int64_t lda, int64_t sa, const float *B, int64_t ldb,
                      int64_t sb) {
    return reinterpret_cast<uintptr_t>(A) % 16 == 0 && reinterpret_cast<uintptr_t>(B) % 16 == 0 &&
           lda % 4 == 0 && ldb % 4 == 0 && sa % 4 == 0 && sb % 4 == 0;
}

// The cost model's "aligned" class: where the direct-load kernels keep
// 16-byte loads.  That takes 16-byte-aligned rows, and edge tiles clamp by
// whole 16-byte groups, which needs the row length of each operand stored
// k-major (N for B as stored, M for A transposed) to be a multiple of 4;
// otherwise those kernels fall back to 4-byte loads, as for unaligned rows.
bool direct_fast(bool rows_aligned, int64_t M, int64_t N, bool ta, bool tb) {
    return rows_aligned && (tb || N % 4 == 0) && (!ta || M % 4 == 0);
}

int run(int variant, int config_id, bool ta, bool tb, int64_t batch, int64_t M, int64_t N,
        int64_t K, const float *A, int64_t lda, int64_t sa, const float *B, int64_t ldb,
        int64_t sb, float *C, int64_t ldc, int64_t sc, void *stream) {
    clear_error();
    int count = 0;
    Plan plan{1, 0, 0, {variant, variant}, {config_id, config_id}};
    if (variant == -1) {  // the library's choice: the products may be split in two launches
        int rc = validate_sizes(M, N, K, lda, ldb, ldc, ta, tb);
        if (rc != GEMM_F32_OK) return rc;
        plan = plan_product(batch, M, N, K, ops_of(ta, tb),
                            direct_fast(operands_aligned(A, lda, sa, B, ldb, sb), M, N, ta, tb));
        variant = plan.variant[0];
        config_id = plan.config[0];
    }
    const ConfigEntry *cfgs = configs_of(variant, &count);
    if (cfgs == nullptr) return fail(GEMM_F32_ENOKERNEL, "unknown variant %d", variant);
    if (config_id < -1 || config_id >= count)
        return fail(GEMM_F32_ENOKERNEL, "variant %d has no configuration %d", variant, config_id);
    int rc = validate(ta, tb, batch, M, N, K, A, lda, sa, B, ldb, sb, C, ldc, sc);
    if (rc != GEMM_F32_OK) return rc;
    if (M == 0 || N == 0 || batch == 0) return GEMM_F32_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (K == 0) {
        err = launch_zero_fill(C, static_cast<int>(M), static_cast<int>(N), ldc,
                               static_cast<int>(batch), sc, s);
    } else {
        if (config_id == -1) {
            int v = 0;
            select_config(batch, M, N, K, &v, &config_id, ops_of(ta, tb),
                          direct_fast(operands_aligned(A, lda, sa, B, ldb, sb), M, N, ta, tb));
            if (v != variant) {  // first configuration of the asked variant that fits
                config_id = 0;
                if (ta || tb)
                    while (config_id + 1 < count && !(cfgs[config_id].caps & kCapTransposed))
                        ++config_id;
            }
        }
        if ((ta || tb) && !(cfgs[config_id].caps & kCapTransposed))
            return fail(GEMM_F32_ENOKERNEL, "configuration %s does not take transposed operands",
                        cfgs[config_id].name);
        const Problem p{static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), A, lda, B,
                        ldb, C, ldc, static_cast<int>(batch), sa, sb, sc, ta, tb};
        if (plan.parts == 1) {
            err = cfgs[config_id].launch(p, s);
        } else {  // the first rows (columns) of C, then the rest: sub-matrices of the operands
            const int split = static_cast<int>(plan.split);
            Problem first = p, rest = p;
            if (plan.axis == 0) {
                first.M = split;
                rest.M = p.M - split;
                rest.A = ta ? A + split : A + static_cast<int64_t>(split) * lda;
                rest.C = C + static_cast<int64_t>(split) * ldc;
            } else {
                first.N = split;
                rest.N = p.N - split;
                rest.B = tb ? B + static_cast<int64_t>(split) * ldb : B + split;
                rest.C = C + split;
            }
            err = cfgs[plan.config[0]].launch(first, s);
            if (err == hipSuccess) err = cfgs[plan.config[1]].launch(rest, s);
        }
    }
    if (err != hipSuccess)
        return fail(GEMM_F32_EHIP, "launch failed: %s", hipGetErrorString(err));
    return GEMM_F32_OK;
}

// gemm_f32_splitk and gemm_f32_splitk_noalloc.  `scratch_of` supplies the
// workspace once the arguments are valid and the bytes it must hold are
// known: the caller's buffer, or the library's static one.
template <class Scratch>
int splitk(int variant, int config_id, int64_t splits, int64_t M, int64_t N, int64_t K,
           const float *A, int64_t lda, const float *B, int64_t ldb, float *C, int64_t ldc,
           Scratch scratch_of, void *stream) {
    if (splits < 0 || splits > 0xffff)
        return fail(GEMM_F32_EINVAL, "splits=%lld outside [0, 65535]", (long long)splits);
    if (splits == 0 && M > 0 && N > 0 && K > 0 && M <= 0x7fffffff && N <= 0x7fffffff &&
        K <= 0x7fffffff)
        splits = auto_splits(M, N, K);
    if (splits == 0) splits = 1;
    if (variant < -1) return fail(GEMM_F32_ENOKERNEL, "unknown variant %d", variant);
    int rc = validate_sizes(M, N, K, lda, ldb, ldc);
    if (rc != GEMM_F32_OK) return rc;
    int64_t used = 1;
    const int len = K > 0 ? split_len(K, splits, &used) : 0;
    if (used <= 1 || M == 0 || N == 0)  // one split: the plain product, no workspace
        return run(variant, variant == -1 ? -1 : config_id, false, false, 1, M, N, K, A, lda, 0, B,
                   ldb, 0, C, ldc, 0, stream);
    rc = validate(false, false, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0);
    if (rc != GEMM_F32_OK) return rc;
    const int64_t need = used * M * N * static_cast<int64_t>(sizeof(float));
    float *W = nullptr;
    rc = scratch_of(need, stream, &W);
    if (rc != GEMM_F32_OK) return rc;
    const Span sw = {reinterpret_cast<uintptr_t>(W), reinterpret_cast<uintptr_t>(W) + need};
    if (overlaps(sw, span_of(A, M, K, lda)) || overlaps(sw, span_of(B, K, N, ldb)) ||
        overlaps(sw, span_of(C, M, N, ldc)))
        return fail(GEMM_F32_EINVAL, "workspace overlaps A, B or C");
    // partial products: a strided batch over the K splits into the workspace
    int v = variant, c = config_id;
    const bool aligned = direct_fast(
        operands_aligned(A, lda, len, B, ldb, static_cast<int64_t>(len) * ldb), M, N, false, false);
    // slices of equal length are a plain batch to the model (a persistent
    // candidate then takes them); a shorter last slice is a split-K launch
    const unsigned sops = K == used * len ? 0u : kOpsSplitK;
    if (v == -1) select_config(used, M, N, len, &v, &c, sops, aligned);
    int count = 0;
    const ConfigEntry *cfgs = configs_of(v, &count);
    if (cfgs == nullptr) return fail(GEMM_F32_ENOKERNEL, "unknown variant %d", v);
    if (c == -1) {
        int vv = 0;
        select_config(used, M, N, len, &vv, &c, sops, aligned);
        if (vv != v) c = 0;
    }
    if (c < 0 || c >= count)
        return fail(GEMM_F32_ENOKERNEL, "variant %d has no configuration %d", v, c);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Problem p{static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), A, lda, B,
                    ldb, W, N, static_cast<int>(used), len, static_cast<int64_t>(len) * ldb,
                    M * N, false, false, len};
    hipError_t err = cfgs[c].launch(p, st);
    if (err == hipSuccess) {
        const bool vec4 = (N % 4) == 0 && (ldc % 4) == 0 &&
                          reinterpret_cast<uintptr_t>(C) % 16 == 0 &&
                          reinterpret_cast<uintptr_t>(W) % 16 == 0;
        const int64_t items = M * (vec4 ? N / 4 : N);
        const unsigned grid = static_cast<unsigned>(std::min<int64_t>((items + 255) / 256, 8192));
        if (vec4)
            hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3(grid), dim3(256), 0, st, W, M * N,
                               static_cast<int>(used), static_cast<int>(M), static_cast<int>(N), C,
                               ldc);
        else
            hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3(grid), dim3(256), 0, st, W, M * N,
                               static_cast<int>(used), static_cast<int>(M), static_cast<int>(N), C,
                               ldc);
        err = hipGetLastError();
    }
    if (err != hipSuccess) return fail(GEMM_F32_EHIP, "launch failed: %s", hipGetErrorString(err));
    return GEMM_F32_OK;
}

// Library-owned scratch of gemm_f32_splitk_noalloc, for callers that
// cannot allocate device memory.  Each device holds its own copy for the
// life of the process.  In host code `scratch` names a host-side stand-in:
// its device address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is passed to
// kernels.  The split-K kernels overwrite every element they later read, so
// nothing needs clearing between calls.
constexpr int64_t kScratchBytes = int64_t{GEMM_F32_SPLITK_SCRATCH_BYTES};
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    float *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch_slots[kMaxDevices];

// Device address of the scratch on the device that runs `stream` (the
// current device for the null stream).
int scratch_address(void *stream, float **out) {
    int current = -1;
    hipError_t err = hipGetDevice(&current);
    if (err != hipSuccess) return fail(GEMM_F32_EHIP, "hipGetDevice: %s", hipGetErrorString(err));
    int dev = current;
    if (stream != nullptr) {
        hipDevice_t d = 0;
        err = hipStreamGetDevice(static_cast<hipStream_t>(stream), &d);
        if (err != hipSuccess)
            return fail(GEMM_F32_EHIP, "hipStreamGetDevice: %s", hipGetErrorString(err));
        dev = static_cast<int>(d);
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(GEMM_F32_EINVAL, "device %d out of range", dev);
    ScratchSlot &slot = g_scratch_slots[dev];
    std::call_once(slot.once, [&] {
        if (dev != current && (slot.err = hipSetDevice(dev)) != hipSuccess) return;
        void *p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess) slot.ptr = static_cast<float *>(p);
        if (dev != current) {
            const hipError_t back = hipSetDevice(current);
            if (slot.err == hipSuccess) slot.err = back;
        }
    });
    if (slot.err != hipSuccess || slot.ptr == nullptr)
        return fail(GEMM_F32_EHIP, "scratch address on device %d: %s", dev,
                    hipGetErrorString(slot.err));
    *out = slot.ptr;
    return GEMM_F32_OK;
}

}  // namespace

hipError_t launch_zero_fill(float *C, int M, int N, int64_t ldc, int batch, int64_t sc,
                            hipStream_t stream) {
    const int64_t total = static_cast<int64_t>(M) * N * batch;
    const int64_t blocks = (total + 255) / 256;
    const unsigned grid = static_cast<unsigned>(blocks < 4096 ? blocks : 4096);
    hipLaunchKernelGGL(zero_fill_kernel, dim3(grid), dim3(256), 0, stream, C, M, N, ldc, batch, sc);
    return hipGetLastError();
}

}  // namespace gemm_f32_impl

using namespace gemm_f32_impl;

extern "C" {

int gemm_f32(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
             int64_t ldb, float *C, int64_t ldc, void *stream) {
    return run(-1, -1, false, false, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, stream);
}

int gemm_f32_variant(int variant, int config_id, int64_t M, int64_t N, int64_t K, const float *A,
                     int64_t lda, const float *B, int64_t ldb, float *C, int64_t ldc,
                     void *stream) {
    if (variant < 0) return (clear_error(), fail(GEMM_F32_ENOKERNEL, "unknown variant %d", variant));
    return run(variant, config_id, false, false, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0,
               stream);
}

int gemm_f32_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const float *A,
                             int64_t lda, int64_t strideA, const float *B, int64_t ldb,
                             int64_t strideB, float *C, int64_t ldc, int64_t strideC,
                             void *stream) {
    clear_error();
    int rc = validate_batch(batch, M, N, K, lda, strideA, ldb, strideB, ldc, strideC);
    if (rc != GEMM_F32_OK) return rc;
    return run(-1, -1, false, false, batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc,
               strideC, stream);
}

int gemm_f32_strided_batched_variant(int variant, int config_id, int64_t batch, int64_t M,
                                     int64_t N, int64_t K, const float *A, int64_t lda,
                                     int64_t strideA, const float *B, int64_t ldb,
                                     int64_t strideB, float *C, int64_t ldc, int64_t strideC,
                                     void *stream) {
    if (variant < 0) return (clear_error(), fail(GEMM_F32_ENOKERNEL, "unknown variant %d", variant));
    return run(variant, config_id, false, false, batch, M, N, K, A, lda, strideA, B, ldb, strideB,
               C, ldc, strideC, stream);
}

int64_t gemm_f32_splitk_workspace_size(int64_t M, int64_t N, int64_t K, int64_t splits) {
    if (M <= 0 || N <= 0 || K <= 0 || splits < 0 || M > 0x7fffffff || N > 0x7fffffff ||
        K > 0x7fffffff || splits > 0xffff)
        return 0;
    if (splits == 0) splits = auto_splits(M, N, K);
    if (splits <= 1) return 0;
    int64_t used = 0;
    split_len(K, splits, &used);
    return used > 1 ? used * M * N * static_cast<int64_t>(sizeof(float)) : 0;
}

int gemm_f32_splitk(int variant, int config_id, int64_t splits, int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda, const float *B, int64_t ldb, float *C,
                    int64_t ldc, void *workspace, int64_t workspace_bytes, void *stream) {
    clear_error();
    auto caller_buffer = [=](int64_t need, void *, float **W) {
        float *w = static_cast<float *>(workspace);
        if (w == nullptr || workspace_bytes < need)
            return fail(GEMM_F32_EINVAL, "workspace of %lld bytes needed, %lld given",
                        (long long)need, (long long)(w ? workspace_bytes : 0));
        if (reinterpret_cast<uintptr_t>(w) % 4)
            return fail(GEMM_F32_EINVAL, "workspace not 4-byte aligned");
        *W = w;
        return GEMM_F32_OK;
    };
    return splitk(variant, config_id, splits, M, N, K, A, lda, B, ldb, C, ldc, caller_buffer,
                  stream);
}

int gemm_f32_splitk_noalloc(int variant, int config_id, int64_t splits, int64_t M, int64_t N,
                            int64_t K, const float *A, int64_t lda, const float *B, int64_t ldb,
                            float *C, int64_t ldc, void *stream) {
    clear_error();
    // library's choice of splits, capped so that the partials fit the scratch
    if (splits == 0 && M > 0 && N > 0 && K > 0 && M <= 0x7fffffff && N <= 0x7fffffff &&
        K <= 0x7fffffff) {
        const int64_t fit = kScratchBytes / (M * N * static_cast<int64_t>(sizeof(float)));
        splits = std::max<int64_t>(1, std::min(auto_splits(M, N, K), fit));
    }
    auto library_scratch = [](int64_t need, void *s, float **W) {
        if (need > kScratchBytes)
            return fail(GEMM_F32_EINVAL,
                        "split-K partials need %lld bytes, above the %lld-byte static scratch",
                        (long long)need, (long long)kScratchBytes);
        return scratch_address(s, W);
    };
    return splitk(variant, config_id, splits, M, N, K, A, lda, B, ldb, C, ldc, library_scratch,
                  stream);
}

int gemm_f32_ex(int variant, int config_id, int opA, int opB, int64_t batch, int64_t M,
                int64_t N, int64_t K, const float *A, int64_t lda, int64_t strideA,
                const float *B, int64_t ldb, int64_t strideB, float *C, int64_t ldc,
                int64_t strideC, void *stream) {
    clear_error();
    if ((opA != GEMM_F32_OP_N && opA != GEMM_F32_OP_T) ||
        (opB != GEMM_F32_OP_N && opB != GEMM_F32_OP_T))
        return fail(GEMM_F32_EINVAL, "opA/opB must be GEMM_F32_OP_N or GEMM_F32_OP_T");
    if (variant < -1) return fail(GEMM_F32_ENOKERNEL, "unknown variant %d", variant);
    const bool ta = opA == GEMM_F32_OP_T, tb = opB == GEMM_F32_OP_T;
    int rc = validate_batch(batch, M, N, K, lda, strideA, ldb, strideB, ldc, strideC);
    if (rc != GEMM_F32_OK) return rc;
    return run(variant, variant == -1 ? -1 : config_id, ta, tb, batch, M, N, K, A, lda, strideA,
               B, ldb, strideB, C, ldc, strideC, stream);
}

const char *gemm_f32_strerror(int code) {
    switch (code) {
        case GEMM_F32_OK: return "success";
        case GEMM_F32_EINVAL: return "invalid argument";
        case GEMM_F32_EHIP: return "HIP runtime error";
        case GEMM_F32_ENOKERNEL: return "no such kernel variant or configuration";
        default: return "unknown error code";
    }
}

const char *gemm_f32_last_error(void) { return g_last_error; }

int gemm_f32_config_count(int variant) {
    int n = 0;
    return configs_of(variant, &n) ? n : GEMM_F32_ENOKERNEL;
}

const char *gemm_f32_config_name(int variant, int config_id) {
    int n = 0;
    const ConfigEntry *c = configs_of(variant, &n);
    if (c == nullptr || config_id < 0 || config_id >= n) return nullptr;
    return c[config_id].name;
}

int gemm_f32_select(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                    int *variant, int *config_id) {
    clear_error();
    int rc = validate_sizes(M, N, K, lda, ldb, ldc);
    if (rc != GEMM_F32_OK) return rc;
    if (variant == nullptr || config_id == nullptr)
        return fail(GEMM_F32_EINVAL, "NULL output pointer");
    const bool fast = direct_fast(lda % 4 == 0 && ldb % 4 == 0, M, N, false, false);
    const Plan plan = plan_product(1, M, N, K, 0u, fast);
    *variant = plan.variant[0];
    *config_id = plan.config[0];
    return GEMM_F32_OK;
}

int gemm_f32_plan(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                  int *parts, int *axis, int64_t *split, int *variant, int *config_id) {
    clear_error();
    int rc = validate_sizes(M, N, K, lda, ldb, ldc);
    if (rc != GEMM_F32_OK) return rc;
    if (!parts || !axis || !split || !variant || !config_id)
        return fail(GEMM_F32_EINVAL, "NULL output pointer");
    const bool fast = direct_fast(lda % 4 == 0 && ldb % 4 == 0, M, N, false, false);
    const Plan plan = plan_product(1, M, N, K, 0u, fast);
    *parts = plan.parts;
    *axis = plan.parts == 2 ? plan.axis : 0;
    *split = plan.parts == 2 ? plan.split : (plan.axis == 0 ? M : N);
    for (int i = 0; i < 2; ++i) {
        variant[i] = plan.variant[i < plan.parts ? i : 0];
        config_id[i] = plan.config[i < plan.parts ? i : 0];
    }
    return GEMM_F32_OK;
}

int gemm_f32_abi_version(void) { return 3; }

}  // extern "C"
