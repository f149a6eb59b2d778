// The dV-only key-owned launch and the query-owned (dQ) launch of the 16-bit backward at
// d = 256.  This unit is compiled with the compiler's own matrix-core products in
// vector-register form: S and dP land in vector registers, where the softmax-gradient
// code reads them, while the dV and dQ products accumulate in AGPRs through their own
// assembly (one wave per SIMD: every vector instruction saved shows in the time).  The
// dK-only launch stays in fa_bwd.hip: its vector registers are full, and it keeps S and
// dP in AGPRs.
#include "fa_bwd.hpp"

namespace fa {

hipError_t launch_bwd16_d256_dv_dq(const BwdProblem &p, float *dq, float *dv, int nsplit,
                                   int tps, hipStream_t stream) {
  hipError_t e;
  if (p.dtype == kBF16) {
    e = run_bwd_dkdv<256, true, kDV>(p, nullptr, dv, nsplit, tps, stream);
    if (e == hipSuccess) e = run_bwd_dq<256, true>(p, dq, nsplit, tps, stream);
  } else {
    e = run_bwd_dkdv<256, false, kDV>(p, nullptr, dv, nsplit, tps, stream);
    if (e == hipSuccess) e = run_bwd_dq<256, false>(p, dq, nsplit, tps, stream);
  }
  return e;
}

}  // namespace fa
