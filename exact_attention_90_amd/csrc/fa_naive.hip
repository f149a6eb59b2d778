// Naive materialised attention: the standard three steps (MUSA SDK guide
// "FlashAttention optimization", "three-step computation"; pwwt.cn Triton tutorial,
// section 1) as three kernels that round-trip S and P through device memory:
//
//   K1  S = scale * Q K^T          written as [B, H, N, N] in the input dtype
//   K2  P = softmax(S) per row     written as [B, H, N, N] in the input dtype (+ LSE)
//   K3  O = P V                    written as [B, H, N, d] float32
//
// It exists only to measure the device-memory traffic the fused kernel avoids.  Every
// kernel accumulates in float32; indices into S and P are 64-bit (B*H*N*N exceeds 2^31
// at the headline shape).  Grids are grid-stride loops capped at kMaxGrid workgroups.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

template <int DT>
struct Elem;
template <>
struct Elem<kF32> {
  using T = float;
  static __device__ __forceinline__ float load(const T *p) { return *p; }
  static __device__ __forceinline__ T cvt(float x) { return x; }
};
template <>
struct Elem<kF16> {
  using T = _Float16;
  static __device__ __forceinline__ float load(const T *p) { return (float)*p; }
  static __device__ __forceinline__ T cvt(float x) { return (_Float16)x; }
};
template <>
struct Elem<kBF16> {
  using T = __bf16;
  static __device__ __forceinline__ float load(const T *p) { return (float)*p; }
  static __device__ __forceinline__ T cvt(float x) { return (__bf16)x; }
};

// ---- K1: scores, 64 x 64 tile per workgroup, 32 x 32 per wave ----------------------
template <int DT, int D>
__global__ __launch_bounds__(256) void naive_scores_kernel(const void *__restrict__ Qv,
                                                           const void *__restrict__ Kv,
                                                           void *__restrict__ Sv, int N, int BH,
                                                           float scale) {
  using E = Elem<DT>;
  using T = typename E::T;
  const T *Q = static_cast<const T *>(Qv);
  const T *K = static_cast<const T *>(Kv);
  T *S = static_cast<T *>(Sv);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, h = lane >> 5, l32 = lane & 31;
  const int nt = (N + 63) / 64;
  const int64_t tiles = int64_t(BH) * nt * nt;
  for (int64_t id = blockIdx.x; id < tiles; id += gridDim.x) {
    const int bh = int(id / (int64_t(nt) * nt));
    const int rem = int(id % (int64_t(nt) * nt));
    const int i0 = (rem / nt) * 64 + 32 * (w >> 1), j0 = (rem % nt) * 64 + 32 * (w & 1);
    const T *Qh = Q + int64_t(bh) * N * D, *Kh = K + int64_t(bh) * N * D;
    const int qi = i0 + l32, kj = j0 + l32;
    f32x16 acc = {};
    if constexpr (DT == kF32) {
#pragma unroll 4
      for (int kc = 0; kc < D / 8; ++kc) {
        f32x4 a = {}, b = {};
        if (qi < N) a = *reinterpret_cast<const f32x4 *>(Qh + int64_t(qi) * D + 8 * kc + 4 * h);
        if (kj < N) b = *reinterpret_cast<const f32x4 *>(Kh + int64_t(kj) * D + 8 * kc + 4 * h);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mma_f32(a[i], b[i], acc);
      }
    } else {
#pragma unroll 4
      for (int kc = 0; kc < D / 16; ++kc) {
        u32x4 a = {}, b = {};
        if (qi < N) a = *reinterpret_cast<const u32x4 *>(Qh + int64_t(qi) * D + 16 * kc + 8 * h);
        if (kj < N) b = *reinterpret_cast<const u32x4 *>(Kh + int64_t(kj) * D + 16 * kc + 8 * h);
        acc = mma16<DT == kBF16>(a, b, acc);
      }
    }
    // C[i][j]: lane holds column j = j0 + l32, rows i0 + 8(r/4) + 4h + r%4
    if (kj < N) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (i < N) S[(int64_t(bh) * N + i) * N + kj] = E::cvt(scale * acc[r]);
      }
    }
  }
}

// ---- K2: row softmax, one workgroup per row ----------------------------------------
__device__ __forceinline__ float block_reduce(float x, bool is_max, float *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    float y = __shfl_xor(x, off);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < 4; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  __syncthreads();
  return r;
}

template <int DT>
__global__ __launch_bounds__(256) void naive_softmax_kernel(const void *__restrict__ Sv,
                                                            void *__restrict__ Pv,
                                                            float *__restrict__ LSE, int N,
                                                            int64_t rows) {
  using E = Elem<DT>;
  using T = typename E::T;
  const T *S = static_cast<const T *>(Sv);
  T *P = static_cast<T *>(Pv);
  __shared__ float red[4];
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const T *srow = S + row * N;
    T *prow = P + row * N;
    float m = -INFINITY;
    for (int j = threadIdx.x; j < N; j += 256) m = fmaxf(m, E::load(srow + j));
    m = block_reduce(m, true, red);
    float z = 0.f;
    for (int j = threadIdx.x; j < N; j += 256) z += expf(E::load(srow + j) - m);
    z = block_reduce(z, false, red);
    const float inv = 1.0f / z;
    for (int j = threadIdx.x; j < N; j += 256) prow[j] = E::cvt(expf(E::load(srow + j) - m) * inv);
    if (threadIdx.x == 0) LSE[row] = m + logf(z);
  }
}

// ---- K3: O = P V, 128 query rows per workgroup, 32 per wave ---------------------------
// O^T = V^T P^T as in the fused kernel: the lane owns one query row; V tiles of 64 keys
// are staged row-major in LDS and read with the transposing load (16-bit inputs).
template <int DT, int D>
__global__ __launch_bounds__(256) void naive_pv_kernel(const void *__restrict__ Pv,
                                                       const void *__restrict__ Vv,
                                                       float *__restrict__ O, int N, int BH) {
  using E = Elem<DT>;
  using T = typename E::T;
  const T *P = static_cast<const T *>(Pv);
  const T *V = static_cast<const T *>(Vv);
  constexpr int OB = D / 32;
  constexpr int ROWB = D * sizeof(T), CPR = ROWB / 16;
  constexpr int BNK = 64;  // keys per V tile
  __shared__ __attribute__((aligned(16))) char vs[BNK * ROWB];
  // fp32 tiles stay plain row-major; 16-bit tiles use the transposing-read swizzle
  auto vaddr = [](int r, int ch) {
    if constexpr (DT == kF32)
      return r * ROWB + ch * 16;
    else
      return r * ROWB + swz_v<CPR>(r, ch) * 16;
  };
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int grp = lane >> 4, j16 = lane & 15;
  const int vrow0 = 4 * (grp >> 1) + (j16 >> 2), vcol0 = 16 * (grp & 1) + 4 * (j16 & 3);
  const int nqt = (N + 127) / 128;
  const int64_t tiles = int64_t(BH) * nqt;
  for (int64_t id = blockIdx.x; id < tiles; id += gridDim.x) {
    const int bh = int(id / nqt), q = int(id % nqt) * 128 + 32 * w + l32;
    const T *Vh = V + int64_t(bh) * N * D;
    const T *prow = P + (int64_t(bh) * N + (q < N ? q : 0)) * N;
    f32x16 o[OB];
#pragma unroll
    for (int e = 0; e < OB; ++e) o[e] = f32x16{};
    for (int j0 = 0; j0 < N; j0 += BNK) {
      __syncthreads();
      for (int cid = tid; cid < BNK * CPR; cid += 256) {
        const int r = cid / CPR, ch = cid % CPR;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (j0 + r < N)
          val = *reinterpret_cast<const u32x4 *>(
              reinterpret_cast<const char *>(Vh + int64_t(j0 + r) * D) + ch * 16);
        lds_write16(vs, vaddr(r, ch), val);
      }
      __syncthreads();
      if constexpr (DT == kF32) {
        // k-step z covers keys j0 + 2z + h; V operand is that key's row, column 32e + l32
#pragma unroll 4
        for (int z = 0; z < BNK / 2; ++z) {
          const int key = 2 * z + h;
          const float pv = (q < N && j0 + key < N) ? prow[j0 + key] : 0.f;
#pragma unroll
          for (int e = 0; e < OB; ++e) {
            const int col = 32 * e + l32;
            const float vv = *reinterpret_cast<const float *>(vs + key * ROWB + col * 4);
            o[e] = mma_f32(vv, pv, o[e]);
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < BNK / 16; ++u) {
          // B operand: P at keys 16u + 8x + 4h + s for slot 4x + s
          uint32_t pw[4];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int kb = j0 + 16 * u + 8 * x + 4 * h;
            u32x2 v2 = {0u, 0u};
            if (q < N) {
              if ((N & 3) == 0 && kb + 3 < N) {  // rows are 8-byte aligned only then
                v2 = *reinterpret_cast<const u32x2 *>(prow + kb);
              } else {
                uint16_t t4[4] = {0, 0, 0, 0};
                for (int s = 0; s < 4; ++s)
                  if (kb + s < N) t4[s] = reinterpret_cast<const uint16_t *>(prow)[kb + s];
                v2 = u32x2{t4[0] | (uint32_t(t4[1]) << 16), t4[2] | (uint32_t(t4[3]) << 16)};
              }
            }
            pw[2 * x] = v2[0];
            pw[2 * x + 1] = v2[1];
          }
          const u32x4 pf = {pw[0], pw[1], pw[2], pw[3]};
#pragma unroll
          for (int e = 0; e < OB; ++e) {
            const int col = 32 * e + vcol0, ch = col >> 3, cb = (col & 7) * 2;
            const int r0 = 16 * u + vrow0, r1 = r0 + 8;
            u32x2 a0 = lds_read_tr(vs, vaddr(r0, ch) + cb);
            u32x2 a1 = lds_read_tr(vs, vaddr(r1, ch) + cb);
            o[e] = mma16<DT == kBF16>(u32x4{a0[0], a0[1], a1[0], a1[1]}, pf, o[e]);
          }
        }
      }
    }
    if (q < N) {
      float *orow = O + (int64_t(bh) * N + q) * D;
#pragma unroll
      for (int e = 0; e < OB; ++e)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4 *>(orow + 32 * e + 8 * g + 4 * h) =
              f32x4{o[e][4 * g], o[e][4 * g + 1], o[e][4 * g + 2], o[e][4 * g + 3]};
    }
  }
}

static int grid_for(int64_t tiles) { return int(tiles < kMaxGrid ? tiles : kMaxGrid); }

template <int DT, int D>
static hipError_t run_naive(const Problem &p, void *s_ws, void *p_ws, hipStream_t stream) {
  const int BH = p.B * p.H;
  const int nt = (p.N + 63) / 64;
  hipLaunchKernelGGL((naive_scores_kernel<DT, D>), dim3(grid_for(int64_t(BH) * nt * nt)),
                     dim3(256), 0, stream, p.q, p.k, s_ws, p.N, BH, p.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = int64_t(BH) * p.N;
  hipLaunchKernelGGL((naive_softmax_kernel<DT>), dim3(grid_for(rows)), dim3(256), 0, stream,
                     s_ws, p_ws, p.lse, p.N, rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqt = (p.N + 127) / 128;
  hipLaunchKernelGGL((naive_pv_kernel<DT, D>), dim3(grid_for(int64_t(BH) * nqt)), dim3(256), 0,
                     stream, p_ws, p.v, p.o, p.N, BH);
  return hipGetLastError();
}

hipError_t launch_naive(const Problem &p, void *s_ws, void *p_ws, hipStream_t stream) {
  switch (p.dtype) {
    case kF16:
      return p.d == 256   ? run_naive<kF16, 256>(p, s_ws, p_ws, stream)
             : p.d == 128 ? run_naive<kF16, 128>(p, s_ws, p_ws, stream)
                          : run_naive<kF16, 64>(p, s_ws, p_ws, stream);
    case kBF16:
      return p.d == 256   ? run_naive<kBF16, 256>(p, s_ws, p_ws, stream)
             : p.d == 128 ? run_naive<kBF16, 128>(p, s_ws, p_ws, stream)
                          : run_naive<kBF16, 64>(p, s_ws, p_ws, stream);
    default:
      return p.d == 256   ? run_naive<kF32, 256>(p, s_ws, p_ws, stream)
             : p.d == 128 ? run_naive<kF32, 128>(p, s_ws, p_ws, stream)
                          : run_naive<kF32, 64>(p, s_ws, p_ws, stream);
  }
}

}  // namespace fa
