// Configurations of the bf16 direct-to-LDS variants with non-square tiles
// that the selector takes by shape, shared by the files that instantiate
// their plain and bf16-output kernels.
//
//  * 128x256 and 256x128 tiles: 4 waves, 3 stages (72 KiB), two workgroups
//    per compute unit (register budget capped at 256 per lane);
//  * 192x256 (8 waves, 2x4 grid, 96x64 per wave) and 256x192 (4x2 grid,
//    64x96 per wave): 3 stages, late barrier; both operands k-contiguous:
//    pair buffers, as for the 256x256 tile;
//  * the two 128x128 rings the selector puts beside the 4-stage one: 2
//    stages (three workgroups per compute unit), and 4 stages with the
//    k-contiguous operand copied two steps at a time into pair buffers.
#pragma once

#include "mfma_dma_gemm.hpp"

namespace dg {

using Dma256x128s3L = DmaConfig<MFMA_BF16_32x32x16, 256, 128, 32, 2, 2, 3, true, PAIR_NONE, 2>;
using Dma128x256s3L = DmaConfig<MFMA_BF16_32x32x16, 128, 256, 32, 2, 2, 3, true, PAIR_NONE, 2>;
using Dma192x256s3L = DmaConfig<MFMA_BF16_32x32x16, 192, 256, 32, 2, 4, 3, true, PAIR_BOTH_KC>;
using Dma256x192s3L = DmaConfig<MFMA_BF16_32x32x16, 256, 192, 32, 4, 2, 3, true, PAIR_BOTH_KC>;
using Dma128x128s2L = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 32, 2, 2, 2, true>;
using Dma128x128s4LPair = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 32, 2, 2, 4, true, PAIR_KC>;
using Dma128x128k64s3L = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 64, 2, 2, 3, true>;

}  // namespace dg
