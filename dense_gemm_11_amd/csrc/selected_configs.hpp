// The direct-to-LDS configurations the kernel selector uses.  Every file that
// instantiates a selected variant (plain, transposed output, bf16 output,
// fused epilogue, stream-K) takes its configuration from here.
//
//  * bf16, 256x256 tiles: 8 waves in a 2x4 grid (128x64 outputs each), two
//    waves per SIMD, three 32-deep stages with the late barrier; both
//    operands k-contiguous: two pair buffers instead of the stage ring.
//  * bf16, 128x128 tiles: 4 waves, four 32-deep stages, late barrier.
//  * fp32, 256x256 tiles: 4 waves, two 32-deep stages; 128x128 tiles: three
//    16-deep stages (both with the late barrier).
#pragma once

#include "mfma_dma_gemm.hpp"

namespace dg {

using SelBf16Big = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 2, 4, 3, true, PAIR_BOTH_KC>;
using SelBf16Mid = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 32, 2, 2, 4, true>;
using SelF32Big = DmaConfig<MFMA_F32_32x32x2, 256, 256, 32, 2, 2, 2, true>;
using SelF32Mid = DmaConfig<MFMA_F32_32x32x2, 128, 128, 16, 2, 2, 3, true>;

}  // namespace dg
