// Instantiation of the 16-bit fused forward kernel for d = 128: eight 32-row waves per
// workgroup (256 query rows), two per SIMD, which halves the K/V tile loads and the
// bfloat16 widening per query row against four waves.
//
// The kernel template also has a form with two 32-row query blocks per wave (RB = 2:
// every K/V operand read from LDS feeds both blocks, the P V products accumulate in the
// matrix-core registers through their own assembly, one wave per SIMD).  This unit is
// compiled with the matrix-core products of the compiler's own choosing in
// vector-register form, which that form needs for its S products.
#include "fa_fwd16.hpp"

namespace fa {

hipError_t launch_fwd16_d128(const Problem &p, float *o, float *lse, int nsplit, int kps,
                             hipStream_t stream, float *stats) {
  if (stats != nullptr)
    return p.dtype == kBF16 ? run16<128, true, 8, 1, true>(p, o, lse, 1, p.N, stream, stats)
                            : run16<128, false, 8, 1, true>(p, o, lse, 1, p.N, stream, stats);
  return p.dtype == kBF16 ? run16<128, true, 8, 1>(p, o, lse, nsplit, kps, stream)
                          : run16<128, false, 8, 1>(p, o, lse, nsplit, kps, stream);
}

}  // namespace fa
