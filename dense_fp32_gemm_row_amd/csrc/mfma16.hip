// Tile configurations of the MFMA kernels (csrc/mfma_kernels.h) with
// 16 x 16 x 4 instructions (v_mfma_f32_16x16x4_f32): four accumulator
// floats per lane and block, so a wavefront holds several independent
// blocks even in small tiles.  Compiled on their own to keep the build
// parallel; gemm_f32_config_name lists them after the 32 x 32 x 2 ones.

#include "mfma_kernels.h"

namespace gemm_f32_impl {
namespace {

const ConfigEntry kMfma16Configs[] = {
    // 16 x 16 x 4 instructions (m16): a w4x1 wavefront's 16 x 64 slice is
    // four independent 16 x 16 accumulator blocks side by side, whose B
    // values of one k are one 16-byte LDS read (interleaved columns); w2x2
    // gives a 32 x 32 slice (2 x 2 blocks, 8-byte B reads).  For the tiles
    // with about one per CU, and with k-groups (k2, k4) for short K.
    {"mfma2d_64x64x32_w4x1_m16_il", launch_mfma<64, 64, 32, 4, 1, -1, 0, 8, 2, true, true, true, 1, 16>, kCapTransposed},
    {"mfma3d_64x64x32_w4x1_m16_il", launch_mfma<64, 64, 32, 4, 1, -1, 0, 8, 3, true, true, true, 1, 16>, kCapTransposed},
    {"mfma2_64x64x32_w4x1_m16_il", launch_mfma<64, 64, 32, 4, 1, -1, 0, 8, 2, false, true, true, 1, 16>, kCapTransposed},
    {"mfma2d_64x64x32_w2x2_m16_il", launch_mfma<64, 64, 32, 2, 2, -1, 0, 8, 2, true, true, true, 1, 16>, kCapTransposed},
    {"mfma2d_64x64x64_w4x1_k2_m16_il", launch_mfma<64, 64, 64, 4, 1, -1, 0, 8, 2, true, true, true, 2, 16>, kCapTransposed},
    {"mfma2_64x64x64_w4x1_k2_m16_il", launch_mfma<64, 64, 64, 4, 1, -1, 0, 8, 2, false, true, true, 2, 16>, kCapTransposed},
    {"mfma2d_64x64x128_w4x1_k4_m16_il", launch_mfma<64, 64, 128, 4, 1, -1, 0, 8, 2, true, true, true, 4, 16>, kCapTransposed},
    {"mfma2_64x64x128_w4x1_k4_m16_il", launch_mfma<64, 64, 128, 4, 1, -1, 0, 8, 2, false, true, true, 4, 16>, kCapTransposed},
    {"mfma2d_128x128x32_w2x2_m16_il", launch_mfma<128, 128, 32, 2, 2, -1, 0, 8, 2, true, true, true, 1, 16>, kCapTransposed},
    {"mfma2d_128x128x32_w4x2_m16_il", launch_mfma<128, 128, 32, 4, 2, -1, 0, 8, 2, true, true, true, 1, 16>, kCapTransposed},
    // register staging with two register sets (loads two K-steps ahead)
    {"mfma2r_64x64x64_w4x1_k2_m16_il", launch_mfma<64, 64, 64, 4, 1, -1, 0, 8, 2, false, true, true, 2, 16, 2>, kCapTransposed},
    // small tiles for products with few output tiles (256^3: 64 or 32 tiles)
    {"mfma2d_16x64x128_w1x1_k4_m16_il", launch_mfma<16, 64, 128, 1, 1, -1, 0, 8, 2, true, true, true, 4, 16>, kCapTransposed},
    // one K-step of 256: a short K runs as a single step after one load
    {"mfma2d_16x16x256_w1x1_k4_m16", launch_mfma<16, 16, 256, 1, 1, -1, 0, 8, 2, true, true, false, 4, 16>, kCapTransposed},
    {"mfma2d_16x32x256_w1x1_k4_m16_il", launch_mfma<16, 32, 256, 1, 1, -1, 0, 8, 2, true, true, true, 4, 16>, kCapTransposed},
    {"mfma2d_16x64x256_w1x1_k4_m16_il", launch_mfma<16, 64, 256, 1, 1, -1, 0, 8, 2, true, true, true, 4, 16>, kCapTransposed},
    {"mfma2d_32x64x64_w2x1_k2_m16_il", launch_mfma<32, 64, 64, 2, 1, -1, 0, 8, 2, true, true, true, 2, 16>, kCapTransposed},
};

}  // namespace

const ConfigEntry *mfma16_configs(int *count) {
    *count = static_cast<int>(sizeof(kMfma16Configs) / sizeof(kMfma16Configs[0]));
    return kMfma16Configs;
}

}  // namespace gemm_f32_impl
