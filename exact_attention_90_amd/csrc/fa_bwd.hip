// Launch of the 16-bit backward pass (kernels in fa_bwd.hpp; d = 128, and the dV and dQ
// launches of d = 256, are compiled in fa_bwd_d128.hip and fa_bwd_d256.hip) and of the
// split backward's slot sums.
#include "fa_bwd.hpp"

namespace fa {

// d = 256: prep and the dK-only key-owned launch here, the dV-only launch and dQ in
// fa_bwd_d256.hip (compiled for S and dP in vector registers)
template <bool BF16>
static hipError_t run_bwd_d256(const BwdProblem &p, float *dq, float *dk, float *dv, int nsplit,
                               int tps, hipStream_t stream) {
  hipError_t e = run_bwd_prep<256, BF16>(p, stream);
  if (e == hipSuccess) e = launch_bwd16_d256_dv_dq(p, dq, dv, nsplit, tps, stream);
  if (e == hipSuccess) e = run_bwd_dkdv<256, BF16, kDK>(p, dk, nullptr, nsplit, tps, stream);
  return e;
}

template <bool BF16>
static hipError_t run_bwd_any(const BwdProblem &p, float *dq, float *dk, float *dv, int nsplit,
                              int tps, hipStream_t stream) {
  return p.d == 256   ? run_bwd_d256<BF16>(p, dq, dk, dv, nsplit, tps, stream)
         : p.d == 128 ? launch_bwd16_d128(p, dq, dk, dv, nsplit, tps, stream)
                      : run_bwd<64, BF16>(p, dq, dk, dv, nsplit, tps, stream);
}

hipError_t launch_bwd(const BwdProblem &p, hipStream_t stream) {
  if (p.dtype == kF32) return launch_bwd32(p, stream);
  const int tiles = (p.N + 63) / 64;
  return p.dtype == kBF16 ? run_bwd_any<true>(p, p.dq, p.dk, p.dv, 1, tiles, stream)
                          : run_bwd_any<false>(p, p.dq, p.dk, p.dv, 1, tiles, stream);
}

// ------------------------------------------------------------------------------------
// Split backward: the key-owned kernel's query tiles and the query-owned kernel's key
// tiles are cut into nsplit ranges (every range non-empty), each range's dQ, dK and dV
// go to their own slot of the partial buffers, and fa_sum_slots adds the slots in slot
// order (so results are bitwise reproducible) into the gradients.  The gradients are
// sums over keys (dQ) or queries (dK, dV) of per-pair terms, so the ranges add.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fa_sum_slots(const float *__restrict__ part,
                                                    float *__restrict__ out, int64_t n4,
                                                    int nsplit) {
  // n4: float4 elements of one slot
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += int64_t(gridDim.x) * 256) {
    f32x4 acc = reinterpret_cast<const f32x4 *>(part)[i];
    for (int g = 1; g < nsplit; ++g) {
      const f32x4 v = reinterpret_cast<const f32x4 *>(part)[g * n4 + i];
      acc = f32x4{acc[0] + v[0], acc[1] + v[1], acc[2] + v[2], acc[3] + v[3]};
    }
    reinterpret_cast<f32x4 *>(out)[i] = acc;
  }
}

hipError_t launch_bwd_split(const BwdProblem &p, float *parts, int nsplit, int tps,
                            hipStream_t stream) {
  const int64_t slot = int64_t(p.B) * p.H * p.N * p.d;  // floats of one slot
  float *pq = parts, *pk = parts + nsplit * slot, *pv = parts + 2 * nsplit * slot;
  hipError_t e = p.dtype == kBF16  ? run_bwd_any<true>(p, pq, pk, pv, nsplit, tps, stream)
                 : p.dtype == kF16 ? run_bwd_any<false>(p, pq, pk, pv, nsplit, tps, stream)
                                   : launch_bwd32_ranges(p, pq, pk, pv, nsplit, tps, stream);
  if (e != hipSuccess) return e;
  const int64_t n4 = slot / 4;
  const int64_t blocks = (n4 + 255) / 256;
  const int grid = int(blocks < 65536 ? blocks : 65536);
  const float *src[3] = {pq, pk, pv};
  float *dst[3] = {p.dq, p.dk, p.dv};
  for (int x = 0; x < 3; ++x) {
    hipLaunchKernelGGL(fa_sum_slots, dim3(grid), dim3(256), 0, stream, src[x], dst[x], n4,
                       nsplit);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fa
