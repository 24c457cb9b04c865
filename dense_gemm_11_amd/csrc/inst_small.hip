// Small-problem variants (one 16x16 output block per workgroup, K split over
// its four waves): fp32 and bf16 operands, fp32 C and D.
#include "small_gemm.hpp"
#include "variants.hpp"

namespace dg {

#define SMALL_FN(T, A_KC, B_KC, WIDE) \
    dg::launch_kernel<small_gemm_kernel<T, float, A_KC, B_KC, WIDE>, 256>
#define SMALL_TABLE(T)                                                                        \
    {{{SMALL_FN(T, false, false, false), SMALL_FN(T, false, true, false)},                   \
      {SMALL_FN(T, true, false, false), SMALL_FN(T, true, true, false)}},                    \
     {{SMALL_FN(T, false, false, true), SMALL_FN(T, false, true, true)},                     \
      {SMALL_FN(T, true, false, true), SMALL_FN(T, true, true, true)}}},                     \
        &dg::occupancy<small_gemm_kernel<T, float, true, false, true>, 256>

const Variant* small_variant_table(int* count)
{
    static const Variant table[] = {
        {"f32_small16x16x16_w4", 0, KIND_SMALL, 16, 16, 16, 256, 4096, 1, 1, SMALL_TABLE(float)},
        {"bf16_small16x16x32_w4", 1, KIND_SMALL, 16, 16, 32, 256, 4096, 1, 1, SMALL_TABLE(bf16_t)},
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
