// Instantiations of the 16-bit fused forward kernel for d = 64 and d = 256, and the
// dispatch over head sizes (d = 128 is compiled in fa_fwd16_d128.hip).  Both use four
// waves per workgroup.  At d = 64 each wave holds two 32-row query blocks (256 rows per
// workgroup, two waves per SIMD): every K and V operand read from LDS feeds both blocks,
// +6 % against one block per wave at three waves per SIMD, bitwise the same output.  At
// d = 256 one 32-row wave already needs more than half of a SIMD's registers.  Compiled with the compiler's own products in vector-register form: at
// d = 256 O sits in AGPRs (its products written as assembly) and S in VGPRs, so S is
// never copied out of AGPRs (+2 % against S in AGPRs, bitwise the same output); the
// d = 64 code does not change.
#include "fa_fwd16.hpp"

namespace fa {

hipError_t launch_fwd16(const Problem &p, float *o, float *lse, int nsplit, int kps,
                        hipStream_t stream, float *stats) {
  const bool bf16 = p.dtype == kBF16;
  if (stats != nullptr) {  // the statistics-recording form (nsplit = 1)
    switch (p.d) {
      case 256:
        return bf16 ? run16<256, true, 4, 1, true>(p, o, lse, 1, p.N, stream, stats)
                    : run16<256, false, 4, 1, true>(p, o, lse, 1, p.N, stream, stats);
      case 128:
        return launch_fwd16_d128(p, o, lse, 1, p.N, stream, stats);
      default:
        return bf16 ? run16<64, true, 4, 2, true>(p, o, lse, 1, p.N, stream, stats)
                    : run16<64, false, 4, 2, true>(p, o, lse, 1, p.N, stream, stats);
    }
  }
  switch (p.d) {
    case 256:
      return bf16 ? run16<256, true, 4, 1>(p, o, lse, nsplit, kps, stream)
                  : run16<256, false, 4, 1>(p, o, lse, nsplit, kps, stream);
    case 128:
      return launch_fwd16_d128(p, o, lse, nsplit, kps, stream, nullptr);
    default:
      return bf16 ? run16<64, true, 4, 2>(p, o, lse, nsplit, kps, stream)
                  : run16<64, false, 4, 2>(p, o, lse, nsplit, kps, stream);
  }
}

}  // namespace fa
