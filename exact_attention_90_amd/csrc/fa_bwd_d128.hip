// Instantiation of the 16-bit backward kernels for d = 128.  This unit is compiled with
// the compiler's own matrix-core products in vector-register form: in the key-owned
// kernel (one wave per SIMD) the S and dP products then land in vector registers, where
// the softmax-gradient code reads them, while the dV and dK products accumulate in AGPRs
// through their own assembly.  The query-owned and prep kernels compile to the same code
// either way.
#include "fa_bwd.hpp"

namespace fa {

hipError_t launch_bwd16_d128(const BwdProblem &p, float *dq, float *dk, float *dv, int nsplit,
                             int tps, hipStream_t stream) {
  return p.dtype == kBF16 ? run_bwd<128, true>(p, dq, dk, dv, nsplit, tps, stream)
                          : run_bwd<128, false>(p, dq, dk, dv, nsplit, tps, stream);
}

}  // namespace fa
