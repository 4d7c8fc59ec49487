// Tile configurations of the MFMA kernels (csrc/mfma_kernels.h) with
// 32 x 32 x 2 instructions, and the registry of every MFMA configuration
// (these, then those of csrc/mfma16.hip and csrc/mfma_regs.hip).

#include <vector>

#include "mfma_kernels.h"

namespace gemm_f32_impl {
namespace {

const ConfigEntry kMfmaConfigs[] = {
    // First kernel: two LDS buffers, one barrier per K-step, padded A rows
    // (pa0 = unpadded, for the bank-conflict counters).
    {"mfma_128x128x16_w2x2_pa4_pb0", launch_mfma<128, 128, 16, 2, 2, 4, 0, 8, 0>, 0},
    {"mfma_128x128x16_w2x2_pa0_pb0", launch_mfma<128, 128, 16, 2, 2, 0, 0, 8, 0>, 0},
    {"mfma_256x256x16_w2x4_pa4_pb0", launch_mfma<256, 256, 16, 2, 4, 4, 0, 8, 0>, 0},
    {"mfma_256x256x32_w2x4_pa4_pb0", launch_mfma<256, 256, 32, 2, 4, 4, 0, 8, 0>, 0},
    {"mfma_256x256x16_w4x4_pa4_pb0", launch_mfma<256, 256, 16, 4, 4, 4, 0, 8, 0>, 0},
    {"mfma_64x64x16_w2x2_pa4_pb0", launch_mfma<64, 64, 16, 2, 2, 4, 0, 8, 0>, 0},
    {"mfma_64x64x32_w2x2_pa4_pb0", launch_mfma<64, 64, 32, 2, 2, 4, 0, 8, 0>, 0},
    // Pipelined kernel, register staging: mfma3 = three LDS buffers, mfma2p =
    // two buffers with the barrier before the last chunk; A rows padded (pa4)
    // or XOR-swizzled (swz); pb8 pads B rows.
    {"mfma3_256x256x16_w4x4_pa4_pb0", launch_mfma<256, 256, 16, 4, 4, 4, 0, 8, 3>, 0},
    {"mfma3_256x256x16_w4x4_swz_pb0", launch_mfma<256, 256, 16, 4, 4, -1, 0, 8, 3>, 0},
    {"mfma3_256x256x16_w4x4_swz_pb8", launch_mfma<256, 256, 16, 4, 4, -1, 8, 8, 3>, 0},
    {"mfma2p_256x256x32_w4x4_swz_pb0", launch_mfma<256, 256, 32, 4, 4, -1, 0, 8, 2, false, true>, kCapTransposed},
    {"mfma3_128x128x16_w2x2_swz_pb0", launch_mfma<128, 128, 16, 2, 2, -1, 0, 8, 3, false, true>, kCapTransposed},
    {"mfma3_64x64x16_w2x2_swz_pb0", launch_mfma<64, 64, 16, 2, 2, -1, 0, 8, 3, false, true>, kCapTransposed},
    // Pipelined kernel, direct global -> LDS loads on full tiles (register
    // staging on edge tiles): mfma3d = three buffers, mfma2d = two buffers,
    // mfma4d = four;
    // 256x128 / 128x256 tiles fit two workgroups per CU at BK = 16; g4 / g16
    // change the column-strip height of the tile order.
    {"mfma3d_256x256x16_w4x4_swz", launch_mfma<256, 256, 16, 4, 4, -1, 0, 8, 3, true>, 0},
    {"mfma3d_256x256x16_w2x4_swz", launch_mfma<256, 256, 16, 2, 4, -1, 0, 8, 3, true>, 0},
    {"mfma3d_256x128x16_w4x2_swz", launch_mfma<256, 128, 16, 4, 2, -1, 0, 8, 3, true>, 0},
    {"mfma3d_128x256x16_w2x4_swz", launch_mfma<128, 256, 16, 2, 4, -1, 0, 8, 3, true, true>, kCapTransposed},
    {"mfma2d_256x256x32_w4x4_swz", launch_mfma<256, 256, 32, 4, 4, -1, 0, 8, 2, true, true>, kCapTransposed},
    {"mfma2d_256x256x32_w4x4_swz_g4", launch_mfma<256, 256, 32, 4, 4, -1, 0, 4, 2, true>, 0},
    {"mfma2d_256x256x32_w4x4_swz_g16", launch_mfma<256, 256, 32, 4, 4, -1, 0, 16, 2, true>, 0},
    {"mfma2d_256x256x32_w2x4_swz", launch_mfma<256, 256, 32, 2, 4, -1, 0, 8, 2, true>, 0},
    {"mfma3d_256x128x32_w4x2_swz", launch_mfma<256, 128, 32, 4, 2, -1, 0, 8, 3, true, true>, kCapTransposed},
    {"mfma3d_128x256x32_w2x4_swz", launch_mfma<128, 256, 32, 2, 4, -1, 0, 8, 3, true>, 0},
    // Interleaved column blocks of B as stored (il): one 8- or 16-byte LDS
    // read per k for the wave's 2 or 4 column blocks, vector C stores.
    {"mfma2d_256x256x32_w4x4_swz_g4_il", launch_mfma<256, 256, 32, 4, 4, -1, 0, 4, 2, true, true, true>, kCapTransposed},
    {"mfma2d_256x256x32_w4x4_swz_g8_il", launch_mfma<256, 256, 32, 4, 4, -1, 0, 8, 2, true, true, true>, kCapTransposed},
    {"mfma2d_256x256x32_w4x2_swz_g4_il", launch_mfma<256, 256, 32, 4, 2, -1, 0, 4, 2, true, true, true>, kCapTransposed},
    {"mfma2d_256x256x32_w2x4_swz_g4_il", launch_mfma<256, 256, 32, 2, 4, -1, 0, 4, 2, true, true, true>, kCapTransposed},
    {"mfma3d_256x128x32_w4x2_swz_il", launch_mfma<256, 128, 32, 4, 2, -1, 0, 8, 3, true, true, true>, kCapTransposed},
    {"mfma3d_128x256x16_w2x4_swz_il", launch_mfma<128, 256, 16, 2, 4, -1, 0, 8, 3, true, true, true>, kCapTransposed},
    {"mfma3_64x128x16_w2x2_swz_il", launch_mfma<64, 128, 16, 2, 2, -1, 0, 8, 3, false, true, true>, kCapTransposed},
    {"mfma2d_256x256x32_w2x4_swz_g8_il", launch_mfma<256, 256, 32, 2, 4, -1, 0, 8, 2, true, true, true>, kCapTransposed},
    // 128 x 128 tiles with direct loads and two buffers (64 KiB: two
    // workgroups per CU).
    {"mfma2d_128x128x32_w2x2_swz_il", launch_mfma<128, 128, 32, 2, 2, -1, 0, 8, 2, true, true, true>, kCapTransposed},
    // K-groups (k4: four groups of 2 x 2 wavefronts, 16 per workgroup, each
    // group a quarter of every K-step): for shapes with about one tile per CU.
    {"mfma2d_64x64x128_w2x2_k4_swz", launch_mfma<64, 64, 128, 2, 2, -1, 0, 8, 2, true, true, false, 4>, kCapTransposed},
    {"mfma2d_64x64x64_w2x2_k4_swz", launch_mfma<64, 64, 64, 2, 2, -1, 0, 8, 2, true, true, false, 4>, kCapTransposed},
    {"mfma3d_64x64x64_w2x2_k4_swz", launch_mfma<64, 64, 64, 2, 2, -1, 0, 8, 3, true, true, false, 4>, kCapTransposed},
    {"mfma4d_64x64x64_w2x2_k4_swz", launch_mfma<64, 64, 64, 2, 2, -1, 0, 8, 4, true, true, false, 4>, kCapTransposed},
    {"mfma2_64x64x64_w2x2_k4_swz", launch_mfma<64, 64, 64, 2, 2, -1, 0, 8, 2, false, true, false, 4>, kCapTransposed},
    {"mfma3_256x256x16_w4x4_swz_g4_il", launch_mfma<256, 256, 16, 4, 4, -1, 0, 4, 3, false, true, true>, kCapTransposed},
    // Register staging with two register sets (mfma2r): each K-step's loads
    // are issued two steps ahead of their LDS store.
    {"mfma2r_64x64x64_w2x2_k4_swz", launch_mfma<64, 64, 64, 2, 2, -1, 0, 8, 2, false, true, false, 4, 32, 2>, kCapTransposed},
};

}  // namespace

const ConfigEntry *mfma_configs(int *count) {
    static const std::vector<ConfigEntry> all = [] {
        std::vector<ConfigEntry> v(std::begin(kMfmaConfigs), std::end(kMfmaConfigs));
        int n16 = 0;
        const ConfigEntry *c16 = mfma16_configs(&n16);
        v.insert(v.end(), c16, c16 + n16);
        int nr = 0;
        const ConfigEntry *cr = mfma_regs_configs(&nr);
        v.insert(v.end(), cr, cr + nr);
        return v;
    }();
    *count = static_cast<int>(all.size());
    return all.data();
}

}  // namespace gemm_f32_impl
