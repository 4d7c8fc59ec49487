"""Host-side models of the edge-tile load schemes in csrc/mfma_kernels.h: the
clamped register staging (OperandTile::init, init_clamp, load_clamped, and
RingTile's split of K into whole K-steps plus a tail), then the 4-byte
direct loads into LDS with range-checked zero fill (rows that are not
16-byte aligned) and the clamped 16-byte direct loads (aligned rows), both
from OperandTile::init and load_direct.

Edge tiles ("Tiled GEMM: Matrix Multiplication in CUDA", section 7.1) must
not read outside an operand, and every element that reaches a stored output
must be the right one.  The kernel does not check elements inside its K
loop; it relies on clamping, and this test checks the clamping rules over a
grid of tile shapes, operand extents, K and leading dimensions:

* every address the K loop loads lies inside the operand's storage,
  (rows - 1) * ld + cols floats;
* every in-range position of a staged tile holds its own element.

The slot mapping restated here: element e = tid + i * NT of a tile with R
rows (row flavour: R rows of BK k values; k-major flavour: BK k rows of R
columns) is stored in 16-byte slots.  Row flavour: row e / (BK / 4), k
column 4 (e % (BK / 4)).  K-major: k row e / (R / 4), column 4 (e % (R / 4)).
"""

import os

import numpy as np
import pytest

# (R, BK, NT): tile extent, K-step, threads of the workgroup -- the staged
# tiles of the configurations (256 x 256 x 16 with 16 wavefronts, 128 x 128 x
# 16 and 64 x 64 x 16 with 4, the 64 x 64 x 64 k-group tile with 16, and an
# 8-wavefront 256 x 256 x 16 tile)
TILES = [(256, 16, 1024), (128, 16, 256), (64, 16, 256), (64, 64, 1024), (256, 16, 512)]
EXTENTS = [1, 3, 4, 5, 63, 65, 255, 257, 774]
KS = [1, 2, 15, 16, 17, 33, 64, 100]


def slots(R, BK, NT, kmajor):
    e = np.arange(R * BK // 4)  # one entry per 16-byte slot (tid + i * NT over all i)
    assert (R * BK) % (4 * NT) == 0
    if kmajor:
        return e // (R // 4), (e % (R // 4)) * 4  # k row, column
    return e // (BK // 4), (e % (BK // 4)) * 4    # row, k column


def clamped_addresses(R, BK, NT, kmajor, rlim, K, ld):
    """Addresses (first float of each 16-byte load) of every K-loop load of
    every tile, and the logical (row, column) each of the 4 floats stands for
    in the staged tile."""
    ro, co = slots(R, BK, NT, kmajor)
    nk = (K - 1) // BK  # whole K-steps in the loop; the step of the last k is the tail
    out = []
    for r0 in range(0, rlim, R):
        if kmajor:
            last = (rlim - 1) & ~3
            col = np.where(r0 + co < rlim, r0 + co, last)
            base = ro * ld + col
        else:
            row = np.where(r0 + ro < rlim, r0 + ro, rlim - 1)
            base = row * ld + co
        for t in range(nk):
            k0 = t * BK
            addr = base + (k0 * ld if kmajor else k0)
            out.append((r0, k0, addr, ro, co))
    return out


def check(R, BK, NT, kmajor, rlim, K, ld):
    rows, cols = (K, rlim) if kmajor else (rlim, K)
    size = (rows - 1) * ld + cols
    n = 0
    for r0, k0, addr, ro, co in clamped_addresses(R, BK, NT, kmajor, rlim, K, ld):
        assert addr.min() >= 0 and addr.max() + 3 < size, (R, BK, kmajor, rlim, K, ld, r0, k0)
        for j in range(4):
            if kmajor:  # position (k row ro + k0, column r0 + co + j)
                valid = r0 + co + j < rlim
                want = (ro + k0) * ld + r0 + co + j
            else:       # position (row r0 + ro, k column k0 + co + j)
                valid = r0 + ro < rlim
                want = (r0 + ro) * ld + k0 + co + j
            assert np.array_equal((addr + j)[valid], want[valid]), (R, BK, kmajor, rlim, K, ld)
        n += addr.size
    return n


@pytest.mark.parametrize("R,BK,NT", TILES)
@pytest.mark.parametrize("kmajor", [True, False], ids=["kmajor", "rows"])
def test_clamped_loads_stay_inside_and_fill_in_range_positions(R, BK, NT, kmajor):
    n = 0
    for rlim in EXTENTS:
        for K in KS:
            width = rlim if kmajor else K
            for ld in sorted({width, width + 3, 4 * ((width + 3) // 4) + 4}):
                if kmajor and ld < 4:
                    continue  # the launcher keeps the checked kernel for these
                n += check(R, BK, NT, kmajor, rlim, K, ld)
    assert n > 0


def test_model_catches_a_missing_tail():
    """Running the K-step of the last k inside the loop (nk = ceil(K / BK))
    would read past the storage of a k-major operand whose last group
    straddles the row end: the model must see that."""
    R, BK, NT, rlim, K, ld = 64, 16, 256, 5, 32, 5
    ro, co = slots(R, BK, NT, True)
    last = (rlim - 1) & ~3
    base = ro * ld + np.where(co < rlim, co, last)
    k0 = (K // BK - 1) * BK  # the last whole step, which holds k = K - 1
    addr = base + k0 * ld
    assert addr.max() + 3 >= (K - 1) * ld + rlim


# --------------------------------------------------------------------------
# 4-byte direct loads into LDS (rows not 16-byte aligned): one float per lane
# and chunk; a lane whose element is out of range gets an offset outside the
# buffer, which the hardware turns into zero.  Restated from
# OperandTile::init (DW) and load_direct.
# --------------------------------------------------------------------------

def dw_tile_ok(R, BK, NW, kmajor):
    return (R * BK // 64) % NW == 0 and ((64 * NW) % R == 0 if kmajor else (64 * NW) % BK == 0)


def swz(m, S):
    # the kernel's shift: log2 S for S = 2, 4, 8, and 4 for every larger S
    log2s = {2: 1, 4: 2, 8: 3}.get(S, 4)
    r = m & 31
    return (r ^ (r >> log2s)) & (S - 1)


def dw_stage(R, BK, NW, kmajor, r0, k0, rlim, K, ld):
    """LDS image of one K-step: the global element offset each position
    receives, -1 for a zero fill."""
    lds = np.full(R * BK, -2, dtype=np.int64)
    step = 64 * NW // R if kmajor else 64 * NW // BK
    jw = (R * BK // 64) // NW
    S = BK // 4
    p_period = 1 if kmajor else 32 // np.gcd(step, 32)
    for w in range(NW):
        f = w * 64 + np.arange(64)
        if kmajor:
            kr, col = f // R, f % R
            off0 = kr * ld + r0 + col
            lim = np.where(r0 + col < rlim, kr, 0x40000000)
        else:
            m = f // BK
            off0 = (r0 + m) * ld
        for j in range(jw):
            pos = (w + j * NW) * 64 + np.arange(64)
            if kmajor:
                off = off0 + (k0 + j * step) * ld
                ok = lim + j * step + k0 < K
            else:
                p = j % p_period
                kc = 4 * (((f % BK) // 4) ^ np.array([swz(x, S) for x in m + p * step])) + f % 4
                off = off0 + j * step * ld + kc + k0
                ok = (r0 + m + j * step < rlim) & (kc + k0 < K)
            assert (lds[pos] == -2).all(), "a position written twice"
            lds[pos] = np.where(ok, off, -1)
    assert (lds != -2).all(), "a position never written"
    return lds


DW_TILES = [(256, 32, 16), (64, 64, 16), (128, 32, 4), (128, 16, 8), (256, 16, 8), (256, 32, 8),
            (64, 128, 16)]


@pytest.mark.parametrize("R,BK,NW", DW_TILES)
@pytest.mark.parametrize("kmajor", [True, False], ids=["kmajor", "rows"])
def test_four_byte_direct_loads_fill_each_position(R, BK, NW, kmajor):
    if not dw_tile_ok(R, BK, NW, kmajor):
        pytest.skip("tile shape not used with 4-byte loads")
    S = BK // 4
    for rlim, K in [(R, BK), (R - 1, BK - 3), (R + 5, 3 * BK + 1), (7, 5)]:
        ld = (K if not kmajor else rlim) + 1
        for r0 in range(0, rlim, R):
            for k0 in range(0, K, BK):
                lds = dw_stage(R, BK, NW, kmajor, r0, k0, rlim, K, ld)
                if kmajor:  # position (k row, column): LD = R
                    krow, col = np.divmod(np.arange(R * BK), R)
                    valid = (k0 + krow < K) & (r0 + col < rlim)
                    want = (k0 + krow) * ld + r0 + col
                else:       # position (row, physical column), logical column via the swizzle
                    row, pc = np.divmod(np.arange(R * BK), BK)
                    lc = 4 * ((pc // 4) ^ np.array([swz(x, S) for x in row])) + pc % 4
                    valid = (r0 + row < rlim) & (k0 + lc < K)
                    want = (r0 + row) * ld + k0 + lc
                assert np.array_equal(lds[valid], want[valid]), (R, BK, NW, kmajor, rlim, K, r0, k0)
                assert (lds[~valid] == -1).all(), (R, BK, NW, kmajor, rlim, K, r0, k0)


# --------------------------------------------------------------------------
# 16-byte direct loads into LDS with 16-byte-aligned rows: each lane moves
# 16 bytes of a 1 KiB chunk; at edge tiles the rows past the extent load the
# last row (row flavour) and the 16-byte groups past it the last group
# (k-major, extent a multiple of 4).  Whole K-steps only.  Restated from
# OperandTile::init (direct, not DW) and load_direct.
# --------------------------------------------------------------------------

def vec_stage(R, BK, NW, kmajor, r0, k0, rlim, ld):
    """Global element offset of each LDS position of one K-step."""
    S = BK // 4
    lds = np.full(R * BK, -2, dtype=np.int64)
    lane = np.arange(64)
    for c in range(R * BK // 256):  # chunk c belongs to wavefront c % NW
        if kmajor:
            f = c * 256 + lane * 4
            col = np.minimum(r0 + f % R, rlim - 4)
            src = (f // R) * ld + col + k0 * ld
        else:
            m = c * (64 // S) + lane // S
            q = (lane % S) ^ np.array([swz(x, S) for x in m])
            row = np.minimum(r0 + m, rlim - 1)
            src = row * ld + 4 * q + k0
        for t in range(4):
            pos = c * 256 + lane * 4 + t
            assert (lds[pos] == -2).all()
            lds[pos] = src + t
    assert (lds != -2).all()
    return lds


VEC_TILES = [(256, 32, 16), (128, 32, 4), (128, 16, 8), (256, 16, 8), (64, 64, 16), (64, 128, 16)]


@pytest.mark.parametrize("R,BK,NW", VEC_TILES)
@pytest.mark.parametrize("kmajor", [True, False], ids=["kmajor", "rows"])
def test_clamped_direct_loads_fill_in_range_positions(R, BK, NW, kmajor):
    S = BK // 4
    for rlim in ([R, R - 4, R + 8, 4, 12] if kmajor else [R, R - 1, R + 5, 1, 7]):
        K = 3 * BK
        ld = (rlim if kmajor else K) + 4
        rows, cols = (K, rlim) if kmajor else (rlim, K)
        size = (rows - 1) * ld + cols
        for r0 in range(0, rlim, R):
            for k0 in range(0, K, BK):
                lds = vec_stage(R, BK, NW, kmajor, r0, k0, rlim, ld)
                assert lds.min() >= 0 and lds.max() < size, (R, BK, kmajor, rlim, r0, k0)
                if kmajor:
                    krow, col = np.divmod(np.arange(R * BK), R)
                    valid = r0 + col < rlim
                    want = (k0 + krow) * ld + r0 + col
                else:
                    row, pc = np.divmod(np.arange(R * BK), BK)
                    lc = 4 * ((pc // 4) ^ np.array([swz(x, S) for x in row])) + pc % 4
                    valid = r0 + row < rlim
                    want = (r0 + row) * ld + k0 + lc
                assert np.array_equal(lds[valid], want[valid]), (R, BK, NW, kmajor, rlim, r0, k0)


# --------------------------------------------------------------------------
# Split-K slices: the partial products run as a strided batch whose product
# b covers k in [b * len, min((b + 1) * len, K)), len a multiple of 32
# (gemm_f32_splitk).  A kernel reads a slice through the K loop its launcher
# picks for the whole launch: without a K check it runs ceil(len_b / BK)
# whole K-steps, so it may only be picked when every slice is whole K-steps.
# Restated from launch_mfma's edge_k rule and RingTile's step counts.
# --------------------------------------------------------------------------

def mfma_bk(name):
    """K-step of an MFMA configuration, from its name (..._BMxBNxBK_...)."""
    import re

    return int(re.search(r"_(\d+)x(\d+)x(\d+)_", name).group(3))


def slice_reads(K, length, used, BK, edge_k):
    """For each slice b, the k range [lo, hi) of the operands that its
    whole-step K loop loads (the partial or clamped tail is zero filled past
    the slice and not counted here)."""
    out = []
    for b in range(used):
        kb = min(length, K - b * length)
        if edge_k:
            nk = kb // BK  # checked kernels: whole steps inside the slice, then a tail
        else:
            nk = -(-kb // BK)  # no K check: every step of the slice is loaded whole
        out.append((b * length, b * length + nk * BK, b * length + kb))
    return out


def _edge_k(K, length, BK):
    return K % BK != 0 or length % BK != 0


@pytest.mark.parametrize("K,splits", [(4160, 4), (1029, 7), (1029, 3), (1024, 4), (65536, 16),
                                      (8192, 3), (777, 2), (4096, 5)])
def test_splitk_slices_stay_inside_their_k_range(K, splits):
    from dense_fp32_gemm_row_amd import binding as b

    if not os.path.exists(b.LIBRARY):
        pytest.skip("library not built")
    b.load()
    M = N = 256
    ws = b.gemm_f32_splitk_workspace_size(M, N, K, splits)
    used = ws // (4 * M * N) if ws else 1
    length = -(-K // splits)
    length = max(32, -(-length // 32) * 32)
    assert used == -(-K // length)
    for name in b.config_names(b.VARIANT_MFMA):
        BK = mfma_bk(name)
        for lo, hi, end in slice_reads(K, length, used, BK, _edge_k(K, length, BK)):
            assert lo <= hi <= end, (name, K, splits, lo, hi, end)


def test_splitk_model_sees_the_unchecked_overrun():
    """The model has teeth: deciding the K check on K alone (K = 4160 is
    whole 64-k steps, the 1056-k slices are not) lets slice 0 read into
    slice 1 and the last slice read past K."""
    K, length, used, BK = 4160, 1056, 4, 64
    reads = slice_reads(K, length, used, BK, K % BK != 0)
    assert reads[0][1] > reads[0][2]
    assert reads[-1][1] > K


# --------------------------------------------------------------------------
# Operands loaded straight into registers (csrc/mfma_regs.hip).  Per chunk c
# of 16 k, lane (g, i) feeds instruction s with k = 16 c + 4 g + s.  Row
# flavour (A as stored, B transposed): block f of the operand is row r_f and
# the lane loads its 4 values of k as one run.  K-major flavour (B as stored,
# A transposed): the lane's F blocks are the F adjacent rows starting at
# base + F i and it loads them as one run per k row.  Rows past the extent
# load the last row (row flavour); a k-major group that starts past it loads
# the group holding the last row.  The loop runs chunks 0 .. (K - 1) / 16 - 1
# (with edges), the chunk of the last k is a checked tail split over the
# groups by instruction, and shapes where a k-major group could pass the
# operand's storage (extent < F - 1) check every element.
# --------------------------------------------------------------------------

# (BM, BN, WM, WN, KG, whole): the register-direct configurations and other
# splits of the same kernel template; whole = False: whole shapes also run the
# clamped kernel (its last chunk a tail)
REGS_TILES = [(64, 64, 1, 1, 4, True), (128, 128, 1, 1, 4, False), (128, 64, 1, 1, 4, True),
              (64, 64, 4, 1, 4, True), (64, 64, 2, 2, 4, True), (32, 64, 1, 1, 8, True),
              (64, 64, 1, 1, 2, True), (64, 64, 1, 1, 1, True), (16, 16, 1, 1, 4, True)]
REGS_SHAPES = [  # M, N, K, ld pad of A, ld pad of B
    (257, 259, 97, 0, 0), (64, 64, 64, 0, 0), (128, 64, 48, 0, 0), (65, 67, 17, 0, 0),
    (1, 1, 1, 0, 0), (3, 2, 5, 0, 0), (70, 3, 33, 2, 0), (5, 2, 100, 0, 0), (64, 1, 16, 0, 0),
    (33, 7, 16, 0, 0), (130, 129, 31, 1, 3), (1, 4, 32, 0, 0), (17, 5, 15, 0, 0), (40, 6, 50, 0, 0),
    (129, 8, 20, 0, 0), (256, 256, 64, 0, 0), (6, 130, 40, 0, 1)]


def regs_operand(kmajor, F, il, base, i, R, clamp):
    """Rows of the lane's F blocks, and the rows its loads use (clamped)."""
    rows = [base + F * i + f if il else base + 16 * f + i for f in range(F)]
    if kmajor:
        r0 = rows[0]
        rc0 = ((R - 1) // F) * F if clamp and r0 > R - 1 else r0
        return rows, [rc0 + f for f in range(F)]
    return rows, [min(r, R - 1) if clamp else r for r in rows]


def regs_model(BM, BN, WM, WN, KG, M, N, K, lda, ldb, whole_ok=True, ta=False, tb=False):
    """Every load of the register-direct kernel as (first float, length), the
    positions that would receive another element than their own, and the k
    values each tile's k-groups cover, restated from the kernel."""
    WTM, WTN = BM // WM, BN // WN
    FM, FN = WTM // 16, WTN // 16
    whole = M % BM == 0 and N % BN == 0 and K % 16 == 0 and whole_ok
    clamp_ok = (not ta or M >= FM - 1) and (tb or N >= FN - 1)
    edge = 0 if whole else (1 if clamp_ok else 2)
    nloop = K // 16 if edge == 0 else ((K - 1) // 16 if edge == 1 else 0)
    nchunks = nloop if edge == 0 else (K + 15) // 16
    # operand: (kmajor, F, interleaved, extent, ld, element address of (row, k))
    opa = (ta, FM, ta, M, lda, (lambda r, k: k * lda + r) if ta else (lambda r, k: r * lda + k))
    opb = (not tb, FN, True, N, ldb, (lambda r, k: r * ldb + k) if tb else (lambda r, k: k * ldb + r))
    loads = {"A": [], "B": []}
    wrong = []
    covered = {}
    for m0 in range(0, M, BM):
        for n0 in range(0, N, BN):
            ks = []
            for kg in range(KG):
                mine = [(c, False) for c in range(nloop) if c % KG == kg]
                ks += [16 * c + q for c, _ in mine for q in range(16)]
                if edge == 2:
                    mine = [(c, True) for c in range(nchunks) if c % KG == kg]
                    ks += [16 * c + q for c, _ in mine for q in range(16) if 16 * c + q < K]
                elif nchunks > nloop and kg < min(KG, 4):
                    ts = min(KG, 4)
                    mine.append((nloop, True))
                    ks += [16 * nloop + 4 * gg + s for gg in range(4) for s in range(4)
                           if s % ts == kg and 16 * nloop + 4 * gg + s < K]
                for wm in range(WM):
                    for wn in range(WN):
                        for name, (kmajor, F, il, R, ld, addr), base in (
                                ("A", opa, m0 + wm * WTM), ("B", opb, n0 + wn * WTN)):
                            for g in range(4):
                                for i in range(16):
                                    rows, used = regs_operand(kmajor, F, il, base, i, R, edge != 0)
                                    for c, checked in mine:
                                        for s in range(4):
                                            k = 16 * c + 4 * g + s
                                            for r, ru in zip(rows, used):
                                                if checked:
                                                    if k < K and r < R:
                                                        loads[name].append((addr(r, k), 1))
                                                    continue  # else zero
                                                if r < R and addr(ru, k) != addr(r, k):
                                                    wrong.append((name, r, k))
                                            if not checked:
                                                if kmajor:
                                                    loads[name].append((addr(used[0], k), F))
                                                elif s == 0:
                                                    loads[name] += [(addr(ru, 16 * c + 4 * g), 4) for ru in used]
            covered[(m0, n0)] = sorted(ks)
    ends = {"A": (K - 1) * lda + M if ta else (M - 1) * lda + K,
            "B": (N - 1) * ldb + K if tb else (K - 1) * ldb + N}
    return loads, wrong, covered, ends


@pytest.mark.parametrize("ops", ["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("tile", REGS_TILES, ids=lambda t: "x".join(map(str, t)))
def test_register_direct_loads_inside_and_complete(tile, ops):
    """Every load of the register-direct kernel lies inside the operands'
    storage ((rows - 1) ld + cols floats, as stored), every position that
    feeds a stored output receives its own element, and each tile's k-groups
    cover every k < K exactly once (the tail's positions past K are zero)."""
    BM, BN, WM, WN, KG, whole_ok = tile
    ta, tb = ops[0] == "T", ops[1] == "T"
    for M, N, K, pa, pb in REGS_SHAPES:
        lda = (M if ta else K) + pa
        ldb = (K if tb else N) + pb
        loads, wrong, covered, ends = regs_model(BM, BN, WM, WN, KG, M, N, K, lda, ldb, whole_ok,
                                                 ta, tb)
        for op in "AB":
            for first, length in loads[op]:
                assert 0 <= first and first + length <= ends[op], (op, ops, tile, (M, N, K), first, length)
        assert not wrong, (ops, tile, (M, N, K), wrong[:3])
        for key, ks in covered.items():
            assert ks == list(range(K)), (ops, tile, (M, N, K), key)


def test_register_direct_model_sees_a_loop_over_the_last_chunk():
    """The check above fails if the loop also ran the chunk of the last k
    with clamped loads (no tail): a group of columns that straddles N then
    reads past the end of B in the last k row."""
    BM, BN, WM, WN, KG, _ = REGS_TILES[0]
    M, N, K = 65, 67, 32  # K whole chunks, N not a multiple of 4
    lda, ldb = K, N
    WTN, FN = BN // WN, BN // WN // 16
    b_end = (K - 1) * ldb + N
    overrun = False
    for n0 in range(0, N, BN):
        for i in range(16):
            bcol = n0 + FN * i
            bcol_c = ((N - 1) // FN) * FN if bcol > N - 1 else bcol
            k = K - 1  # the last k row, loaded unchecked
            overrun |= k * ldb + bcol_c + FN > b_end
    assert overrun


def xcd_remap(bid, n):
    """Restated from csrc/gemm_internal.h: hardware workgroup id -> logical
    id, consecutive logical ids on one XCD (workgroup b runs on XCD b % 8)."""
    q, r = divmod(n, 8)
    xcd, local = bid % 8, bid // 8
    return xcd * (q + 1) + local if xcd < r else r * (q + 1) + (xcd - r) * q + local


@pytest.mark.parametrize("grid", [1, 7, 8, 100, 255, 256])
def test_persistent_walk_covers_every_tile_once(grid):
    """The persistent register-direct kernel: workgroup b of `grid` takes
    logical tiles xcd_remap(b, grid) + j * grid while they are below the
    tile count; every tile is taken by exactly one workgroup, for tile counts
    below, at and above the grid."""
    for total in sorted({grid, max(1, grid - 3), grid + 1, 2 * grid, 5 * grid + 3}):
        g = min(grid, total)  # the launcher never starts more workgroups than tiles
        seen = []
        for b in range(g):
            logical = xcd_remap(b, g)
            while logical < total:
                seen.append(logical)
                logical += g
        assert sorted(seen) == list(range(total)), (grid, total)


# --------------------------------------------------------------------------
# the persistent register-direct tile's buffer loads (BufOperand), whole and
# edge forms, restated with numpy over the 64 lanes
# --------------------------------------------------------------------------

OUT = 1 << 31  # a lane offset past the resource: the load returns zeros


def buf_offsets(kmajor, F, il, base, R, ld, K, c, q, edge, kchk):
    """Lane byte offsets (voffset + soffset) of piece q of chunk c, and for
    each of the 4 floats of every lane's 16-byte load the operand element
    (row, k) it stands for; (row-flavour piece q is block q, k-major piece q
    is k row q, which loads F / 4 pieces of 4 floats and, when F % 4 == 2,
    one of 2)."""
    lane = np.arange(64)
    g, i = lane // 16, lane % 16
    out = []
    if kmajor:
        # runs of F floats: pieces of 4, then one of 2 when F % 4 == 2
        for p in range(0, F, 4):
            width = min(4, F - p)
            col = base + F * i + p
            v = np.where(col < R, (4 * g * ld + F * i + p) * 4, OUT) if edge else (4 * g * ld + F * i + p) * 4
            k = 16 * c + 4 * g + q
            if edge and kchk:
                v = np.where(k < K, v, OUT)
            off = np.where(v >= OUT, OUT, v + q * ld * 4)
            out.append((off, [(col + e, k) for e in range(width)]))
    else:
        r = base + (F * i + q if il else 16 * q + i)
        v = np.where(r < R, ((r - base) * ld + 4 * g) * 4, OUT) if edge else ((r - base) * ld + 4 * g) * 4
        if edge and kchk:
            v = np.where(16 * c < K - 4 * g, v, OUT)
        out.append((v, [(r, 16 * c + 4 * g + e) for e in range(4)]))
    return out


def persistent_model(M, N, K, lda, ldb, ta, tb, BM=128, BN=128, KG=4, D=2, no_kchk=False):
    """Every load of the persistent kernel: checks that a load with a lane
    offset inside the resource reads, for each of its floats, the element
    its position stands for, inside the operand's storage; that positions
    past M, N or K read zeros (offset past the resource) or, in the rounds
    that do not check k, never occur; and that each tile's groups cover every
    k < K once.  no_kchk: a planted mistake, no round checks k.  Returns
    the number of loads checked."""
    whole = M % BM == 0 and N % BN == 0 and K % (16 * KG * D) == 0
    edge = not whole
    assert not edge or (K % 4 == 0 and (not ta or M % 4 == 0) and (tb or N % 4 == 0))
    FM, FN = BM // 16, BN // 16
    ng = -(-(-(-K // 16)) // (KG * D)) * D if edge else K // 16 // KG
    # operand: (kmajor, F, interleaved, extent, ld, element index of (row, k), storage floats)
    opa = (ta, FM, ta, M, lda, (lambda r, k: k * lda + r) if ta else (lambda r, k: r * lda + k),
           (K - 1) * lda + M if ta else (M - 1) * lda + K)
    opb = (not tb, FN, True, N, ldb, (lambda r, k: r * ldb + k) if tb else (lambda r, k: k * ldb + r),
           (N - 1) * ldb + K if tb else (K - 1) * ldb + N)
    nloads = 0
    for kg in range(KG):
        chunk_of = lambda t: kg + KG * t  # noqa: E731
        t_chk = ng
        if edge:
            t_chk = 0
            while t_chk + D < ng and 16 * chunk_of(t_chk + 2 * D - 1) + 16 <= K:
                t_chk += D
        # (chunk, checked): the first D chunks (checked in the edge form), then
        # round t's loads of chunks t + u + D
        loads = [(chunk_of(u), edge) for u in range(D)]
        for t in range(0, ng - D, D):
            loads += [(chunk_of(t + u + D), edge and t >= t_chk) for u in range(D)]
        for m0 in range(0, M, BM):
            for n0 in range(0, N, BN):
                for (kmajor, F, il, R, ld, index, size), base in ((opa, m0), (opb, n0)):
                    origin = lambda c: base + 16 * c * ld if kmajor else base * ld + 16 * c  # noqa: E731
                    for c, kchk in loads:
                        for q in range(4 if kmajor else F):
                            for off, elems in buf_offsets(kmajor, F, il, base, R, ld, K, c, q, edge,
                                                          kchk and not no_kchk):
                                nloads += 1
                                for e, (r, k) in enumerate(elems):
                                    inside = off < OUT
                                    valid = (r < R) & (k < K)
                                    # a position past M, N or K reads zeros
                                    assert not np.any(inside & ~valid), (kmajor, c, q, e)
                                    idx = origin(c) + off // 4 + e
                                    want = index(r, k)
                                    assert np.all(np.where(inside, idx == want, True)), (kmajor, c, q, e)
                                    assert np.all(np.where(inside, (idx >= 0) & (idx < size), True))
                                    assert np.all(np.where(inside, off + 4 * e < (1 << 31), True))
                                    # a valid position is loaded (not zero-filled)
                                    assert np.all(np.where(valid, inside, True)), (kmajor, c, q, e)
    chunks = [kg + KG * t for kg in range(KG) for t in range(ng)]
    assert sorted(16 * c + j for c in chunks for j in range(16) if 16 * c + j < K) == list(range(K))
    return nloads


PERSISTENT_BUF_SHAPES = [  # M, N, K, ld pads
    (128, 128, 128, 0, 0), (256, 128, 384, 4, 8), (130, 132, 100, 0, 0), (300, 260, 388, 3, 0),
    (4, 4, 20, 0, 0), (128, 132, 4, 0, 4), (129, 256, 256, 0, 0), (192, 256, 512, 0, 0),
    (96, 128, 256, 0, 4)]


PERSISTENT_TILES = [(128, 128, 2), (96, 128, 2)]  # BM, BN, D of the persistent configurations


@pytest.mark.parametrize("tile", PERSISTENT_TILES, ids=lambda t: f"{t[0]}x{t[1]}_d{t[2]}")
@pytest.mark.parametrize("ops", ["NN", "NT", "TN", "TT"])
def test_persistent_buffer_loads(ops, tile):
    """The persistent tile's buffer loads, whole and edge forms: in-range
    lanes read their own element inside the operand, positions past M, N or
    K read zeros through an offset past the resource, and the groups cover
    every k once.  Shapes neither form takes (the edge form needs K, and a
    k-major row length with its per-lane run, multiples of 4) are skipped,
    as the launcher skips them."""
    BM, BN, D = tile
    FM, FN = BM // 16, BN // 16
    ta, tb = ops[0] == "T", ops[1] == "T"
    ran = 0
    for M, N, K, pa, pb in PERSISTENT_BUF_SHAPES:
        whole = M % BM == 0 and N % BN == 0 and K % (64 * D) == 0
        edge_ok = (K % 4 == 0 and (not ta or (M % 4 == 0 and FM % 4 == 0))
                   and (tb or (N % 4 == 0 and FN % 4 == 0)))
        if not whole and not edge_ok:
            continue
        lda = (M if ta else K) + pa
        ldb = (K if tb else N) + pb
        ran += persistent_model(M, N, K, lda, ldb, ta, tb, BM=BM, BN=BN, D=D) > 0
    assert ran >= (1 if ta and FM % 4 else 5)


def test_persistent_buffer_model_sees_an_unchecked_tail():
    """The model fails if no round checked k: a K that is not whole rounds
    then has loads of k past K from memory."""
    persistent_model(128, 128, 100, 100, 128, False, False)
    with pytest.raises(AssertionError):
        persistent_model(128, 128, 100, 100, 128, False, False, no_kchk=True)
