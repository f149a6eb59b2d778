// Internal launch interface between the C boundary (fa_api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the boundary: shapes
// positive, d in {64, 128, 256}, pointers non-null and aligned, grid within limits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace fa {

enum Dtype { kF32 = 0, kF16 = 1, kBF16 = 2 };

struct Problem {
  const void *q, *k, *v;
  float *o, *lse;
  int B, H, N, d;
  float scale;
  int dtype;
};

// Query rows per workgroup of the fused kernels: waves x 32 rows.  kFusedBM (4 waves) is
// the smallest workgroup any fused kernel uses, so it bounds the grid of all of them.
constexpr int kFusedBM = 128;
// Largest grid (in workgroups) any launcher issues: 256 threads x 2^24 < 2^32 work-items.
constexpr int64_t kMaxGrid = int64_t(1) << 24;
// Largest [N, d] slice of one head, in bytes: kernels address a head with 32-bit byte
// offsets and may read one tile (<= 64 KiB) past its end (those reads return zeros).
constexpr int64_t kMaxHeadBytes = (int64_t(1) << 31) - (int64_t(1) << 17);

// Backward pass: inputs, outputs and the caller's workspace split into its three parts
// (dO rounded to the input type, lse2 = LSE log2(e), D = rowsum(dO O)).
struct BwdProblem {
  const void *q, *k, *v;
  const float *o, *lse, *dout;
  float *dq, *dk, *dv;
  void *ws_do16;
  float *ws_lse2, *ws_d;
  int B, H, N, d;
  float scale;
  int dtype;
};

// Raises kernel Kern's dynamic-LDS limit to `bytes` on the current device, once per
// device (ids 0..63; beyond that on every call) and process: the limit is a per-device
// attribute, so a process that uses several GPUs sets it on each.  A failure is
// returned and nothing is remembered, so the next call tries again.
template <auto Kern>
inline hipError_t allow_lds_on_device(int bytes) {
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  const hipError_t g = hipGetDevice(&dev);
  if (g != hipSuccess) return g;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(Kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Workgroups of kernel Kern (nt threads, lds bytes of LDS) the current device holds at
// once: compute units x resident workgroups per compute unit, found once per device (ids
// 0..63; beyond that on every call).  0 when the device cannot say.
template <auto Kern>
inline int resident_workgroups(int nt, int lds) {
  static std::atomic<int> known[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const bool cached = dev >= 0 && dev < 64;
  if (cached) {
    const int v = known[dev].load(std::memory_order_acquire);
    if (v > 0) return v;
  }
  int ncu = 0, per = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipFuncSetAttribute(reinterpret_cast<const void *>(Kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, Kern, nt, size_t(lds)) != hipSuccess)
    return 0;
  const int v = ncu * per;
  if (cached && v > 0) known[dev].store(v, std::memory_order_release);
  return v > 0 ? v : 0;
}

hipError_t launch_fused(const Problem &p, hipStream_t stream);
// the 16-bit kernels (binary16 / bfloat16 inputs): key ranges as in launch_fused_split,
// written to o and lse (nsplit = 1, kps = N: the attention itself); d = 128 lives in
// its own compilation unit.  stats != nullptr selects the statistics-recording form
// (nsplit = 1; see launch_fused_stats).
hipError_t launch_fwd16(const Problem &p, float *o, float *lse, int nsplit, int kps,
                        hipStream_t stream, float *stats = nullptr);
hipError_t launch_fwd16_d128(const Problem &p, float *o, float *lse, int nsplit, int kps,
                             hipStream_t stream, float *stats);
// the fused forward in its statistics-recording form: besides O and LSE, every query
// row's running max (base-2 units, scale log2(e) max s) and running row sum after every
// 64-key tile, as float pairs [B H N][ceil(N / 64)][2]
hipError_t launch_fused_stats(const Problem &p, float *stats, hipStream_t stream);
// nsplit key ranges of kps keys into the partial buffers (opart: nsplit
// slots of B H N d floats, lpart: nsplit slots of B H N floats), then merged into p.o, p.lse
hipError_t launch_fused_split(const Problem &p, float *opart, float *lpart, int nsplit,
                              int kps, hipStream_t stream);
hipError_t launch_bwd(const BwdProblem &p, hipStream_t stream);    // every dtype
// the 16-bit backward at d = 128 (fa_bwd_d128.hip): nsplit ranges of tps tiles each
hipError_t launch_bwd16_d128(const BwdProblem &p, float *dq, float *dk, float *dv, int nsplit,
                             int tps, hipStream_t stream);
// the dV-only and dQ launches of the 16-bit backward at d = 256 (fa_bwd_d256.hip)
hipError_t launch_bwd16_d256_dv_dq(const BwdProblem &p, float *dq, float *dv, int nsplit,
                                   int tps, hipStream_t stream);
// nsplit ranges of tps tiles (64 rows) each; parts holds 3 nsplit slots of
// B H N d floats (dQ slots, then dK, then dV), summed into p.dq, p.dk, p.dv
hipError_t launch_bwd_split(const BwdProblem &p, float *parts, int nsplit, int tps,
                            hipStream_t stream);
hipError_t launch_bwd32(const BwdProblem &p, hipStream_t stream);  // fp32 inputs
// fp32 inputs, nsplit ranges of tps 64-row tiles into dq, dk, dv (nsplit slots each)
hipError_t launch_bwd32_ranges(const BwdProblem &p, float *dq, float *dk, float *dv, int nsplit,
                               int tps, hipStream_t stream);
hipError_t launch_naive(const Problem &p, void *s_ws, void *p_ws, hipStream_t stream);

}  // namespace fa
