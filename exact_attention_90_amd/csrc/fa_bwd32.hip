// Attention backward pass for fp32 inputs (gfx950): dQ, dK and dV on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32).
//
// The method and the three-kernel split are those of the 16-bit backward pass
// (fa_bwd.hip; pwwt.cn Triton tutorial, sections 2.4 and 4.4: P recomputed from LSE,
// then the chain rule).  Here nothing is rounded below fp32: dO is used as given, P and
// dS stay fp32.
//
// Operand layout of the fp32 matrix core: A lane holds A[lane % 32][h], B lane holds
// B[h][lane % 32] (h = lane / 32), C as for the 16-bit products.  A k-step over d takes
// columns 8kc + 4h + i (i = 0..3) from one 16-byte chunk per lane half, on both operands.
// A k-step over rows (queries for dV and dK, keys for dQ) takes, in register r of the
// C layout, row 8(r/4) + 4h + r%4 on lane half h: the operand of the other side is one
// 4-byte element of that row, read from LDS.
#include "fa_internal.h"
#include "fa_softmax.hpp"

namespace fa {

// ------------------------------------------------------------------------------------
// prep: per row, D = <dO, O> and lse2 = LSE log2(e)
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void fa_bwd32_prep_kernel(const float *__restrict__ O,
                                                            const float *__restrict__ dO,
                                                            const float *__restrict__ LSE,
                                                            float *__restrict__ lse2,
                                                            float *__restrict__ Dv, int64_t rows) {
  constexpr int TPR = D / 4;
  const int64_t total = rows * TPR;
  for (int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x; gid - threadIdx.x < total;
       gid += int64_t(gridDim.x) * 256) {
    const int64_t row = gid / TPR;
    const int c = int(gid % TPR);
    float part = 0.f;
    if (row < rows) {
      const f32x4 o = *reinterpret_cast<const f32x4 *>(O + row * D + 4 * c);
      const f32x4 g = *reinterpret_cast<const f32x4 *>(dO + row * D + 4 * c);
      part = o[0] * g[0] + o[1] * g[1] + o[2] * g[2] + o[3] * g[3];
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (row < rows && c == 0) {
      Dv[row] = part;
      lse2[row] = LSE[row] * kLog2e;
    }
  }
}

template <int D>
struct CfgB32 {
  static constexpr int NT = 256;               // four waves
  static constexpr int BR = 128;               // resident rows per workgroup (32 per wave)
  static constexpr int BT = 64;                // rows per streamed tile
  static constexpr int ROWB = 4 * D;
  static constexpr int CPR = ROWB / 16;
  static constexpr int TILEB = BT * ROWB;
  static constexpr int CPT = TILEB / 16 / NT;
  static constexpr int KC = D / 8;             // 16-byte chunks per lane half (4 k-steps each)
  static constexpr int OB = D / 32;
  static constexpr int RSTEP = NT / CPR;
  static constexpr int STATB = 1024;
  static constexpr int LDS = 4 * TILEB + 4 * STATB;
  static_assert(CPT >= 1 && TILEB % (16 * NT) == 0, "a tile is whole chunks per thread");
  static_assert(32 * D * 4 <= LDS / 4, "a wave's output rows fit its LDS share");
};

// Tile rows are swizzled per 16-byte chunk: logical chunk ch of row r sits at chunk
// ch ^ (r % 16).  The 32 rows of a row read (one chunk each) then spread over the banks;
// a 4-byte element read touches one chunk of each of two rows per lane half.
__device__ __forceinline__ int el_off32(int row, int col, int rowb) {
  return row * rowb + (((col >> 2) ^ (row & 15)) << 4) + (col & 3) * 4;
}

// loads of a tile into LDS (chunk i of thread tid is LDS chunk i NT + tid): the source
// offset of each chunk, swizzle included (rows of a thread are RSTEP apart)
template <typename C>
__device__ __forceinline__ int dma_src32(int tid, int i) {
  const int row = i * C::RSTEP + tid / C::CPR, ch = tid % C::CPR;
  return row * C::ROWB + ((ch ^ (row & 15)) << 4) - i * C::NT * 16;
}

// ------------------------------------------------------------------------------------
// dkdv: dK and dV of 32 keys per wave
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void fa_bwd32_dkdv_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ dO, const float *__restrict__ lse2, const float *__restrict__ Dv,
    float *__restrict__ dK, float *__restrict__ dV, int N, int nkb, int G, float c, float scale,
    int nsplit, int tps) {
  using C = CfgB32<D>;
  constexpr int KC = C::KC, OB = C::OB, CPT = C::CPT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char *const Qs = smem;
  char *const Gs = smem + 2 * C::TILEB;
  char *const Ls = smem + 4 * C::TILEB;
  char *const Ds = Ls + 2 * C::STATB;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // key block L % nkb, query-tile range (L / nkb) % nsplit, head L / (nkb nsplit); the
  // range's dK and dV go to its slot (as in the 16-bit kernel)
  const int L = xcd_remap(blockIdx.x, G);
  const int rg = (L / nkb) % nsplit, bh = L / nkb / nsplit, k0 = (L % nkb) * C::BR;
  const int64_t hoff = int64_t(bh) * N * D;
  const int64_t slot = int64_t(G / (nkb * nsplit)) * N * D * rg;
  const uint32_t head_bytes = uint32_t(N) * C::ROWB;
  const auto qrs = make_rsrc(Q + hoff, head_bytes);
  const auto grs = make_rsrc(dO + hoff, head_bytes);
  const auto krs = make_rsrc(K + hoff, head_bytes);
  const auto vrs = make_rsrc(V + hoff, head_bytes);
  const auto lrs = make_rsrc(lse2 + int64_t(bh) * N, uint32_t(N) * 4);
  const auto drs = make_rsrc(Dv + int64_t(bh) * N, uint32_t(N) * 4);

  const int key = k0 + 32 * w + l32;
  f32x4 kf[KC], vf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    kf[kc] = __builtin_bit_cast(f32x4, buf_load16(krs, key * C::ROWB + (2 * kc + h) * 16, 0));
    vf[kc] = __builtin_bit_cast(f32x4, buf_load16(vrs, key * C::ROWB + (2 * kc + h) * 16, 0));
  }

  constexpr int ST_STEP = C::NT * 16;
  const int dma_wave = wu * 1024;
  auto load_tile = [&](int stage, int qt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int src = dma_src32<C>(tid, i);
      buf_load16_lds(qrs, Qs + stage * C::TILEB + dma_wave + i * ST_STEP, src,
                     qt * C::TILEB + i * ST_STEP);
      buf_load16_lds(grs, Gs + stage * C::TILEB + dma_wave + i * ST_STEP, src,
                     qt * C::TILEB + i * ST_STEP);
    }
    if (wu == 0) buf_load16_lds(lrs, Ls + stage * C::STATB, lane * 16, qt * 256);
    if (wu == 3) buf_load16_lds(drs, Ds + stage * C::STATB, lane * 16, qt * 256);
  };

  f32x16 dk[OB], dv[OB];
#pragma unroll
  for (int e = 0; e < OB; ++e) dk[e] = dv[e] = f32x16{};

  const int qt0 = rg * tps;                                // first query tile
  const int nqt = min((N + C::BT - 1) / C::BT - qt0, tps);  // tiles of the range
  load_tile(0, qt0);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  lds_barrier();
  for (int qt = 0; qt < nqt; ++qt) {  // qt counts the range's tiles
    const int st = qt & 1;
    if (qt + 1 < nqt) load_tile(st ^ 1, qt0 + qt + 1);
    const char *qs = Qs + st * C::TILEB, *gs = Gs + st * C::TILEB;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // S = Q K^T and dP = dO V^T: queries 32t + (8(r/4) + 4h + r%4), key l32
      f32x16 s = {}, dp = {};
      const int qr = 32 * t + l32;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int off = qr * C::ROWB + (((2 * kc + h) ^ (qr & 15)) << 4);
        const f32x4 qa = *reinterpret_cast<const f32x4 *>(qs + off);
        const f32x4 ga = *reinterpret_cast<const f32x4 *>(gs + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s = mma_f32(qa[i], kf[kc][i], s);
          dp = mma_f32(ga[i], vf[kc][i], dp);
        }
      }
      float p[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qo = (32 * t + 8 * g + 4 * h) * 4;
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(Ls + st * C::STATB + qo);
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(Ds + st * C::STATB + qo);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int r = 4 * g + s4;
          p[r] = ex2(fmaf(s[r], c, -l4[s4]));
          ds[r] = p[r] * (dp[r] - d4[s4]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS, one query pair per step: register r holds
      // query 32t + 8(r/4) + 4h + r%4 on lane half h; the other operand is that query's
      // row at column 32e + l32
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int e = 0; e < OB; ++e) {
          const int off = el_off32(q, 32 * e + l32, C::ROWB);
          dv[e] = mma_f32(*reinterpret_cast<const float *>(gs + off), p[r], dv[e]);
          dk[e] = mma_f32(*reinterpret_cast<const float *>(qs + off), ds[r], dk[e]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    lds_barrier();
  }

  constexpr int WAVE_LDS = (C::LDS / 4) & ~15;
  const int row0 = k0 + 32 * w;
  char *region = smem + w * WAVE_LDS;
  store_rows_lds<D, 1, false>(dk, 0.f, 1.f, 0.5f / scale, region, dK + slot + hoff + int64_t(row0) * D,
                              nullptr, lane, N - row0);
  store_rows_lds<D, 1, false>(dv, 0.f, 1.f, 0.5f, region, dV + slot + hoff + int64_t(row0) * D, nullptr,
                              lane, N - row0);
}

// ------------------------------------------------------------------------------------
// dq: dQ of 32 queries per wave
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, D >= 128 ? 1 : 2) void fa_bwd32_dq_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ dO, const float *__restrict__ lse2, const float *__restrict__ Dv,
    float *__restrict__ dQ, int N, int nqb, int G, float c, float scale, int nsplit, int tps) {
  using C = CfgB32<D>;
  constexpr int KC = C::KC, OB = C::OB, CPT = C::CPT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char *const Ks = smem;
  char *const Vs = smem + 2 * C::TILEB;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // query block L % nqb, key-tile range (L / nqb) % nsplit, head L / (nqb nsplit)
  const int L = xcd_remap(blockIdx.x, G);
  const int rg = (L / nqb) % nsplit, bh = L / nqb / nsplit, q0 = (L % nqb) * C::BR;
  const int64_t hoff = int64_t(bh) * N * D;
  const int64_t slot = int64_t(G / (nqb * nsplit)) * N * D * rg;
  const uint32_t head_bytes = uint32_t(N) * C::ROWB;
  const auto qrs = make_rsrc(Q + hoff, head_bytes);
  const auto grs = make_rsrc(dO + hoff, head_bytes);
  const auto krs = make_rsrc(K + hoff, head_bytes);
  const auto vrs = make_rsrc(V + hoff, head_bytes);

  const int row = q0 + 32 * w + l32;
  f32x4 qf[KC], gf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    qf[kc] = __builtin_bit_cast(f32x4, buf_load16(qrs, row * C::ROWB + (2 * kc + h) * 16, 0));
    gf[kc] = __builtin_bit_cast(f32x4, buf_load16(grs, row * C::ROWB + (2 * kc + h) * 16, 0));
  }
  const float my_lse2 = row < N ? lse2[int64_t(bh) * N + row] : 0.f;
  const float my_d = row < N ? Dv[int64_t(bh) * N + row] : 0.f;

  constexpr int ST_STEP = C::NT * 16;
  const int dma_wave = wu * 1024;
  auto load_tile = [&](int stage, int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int src = dma_src32<C>(tid, i);
      buf_load16_lds(krs, Ks + stage * C::TILEB + dma_wave + i * ST_STEP, src,
                     kt * C::TILEB + i * ST_STEP);
      buf_load16_lds(vrs, Vs + stage * C::TILEB + dma_wave + i * ST_STEP, src,
                     kt * C::TILEB + i * ST_STEP);
    }
  };

  f32x16 dq[OB];
#pragma unroll
  for (int e = 0; e < OB; ++e) dq[e] = f32x16{};

  const int kt0 = rg * tps;                                // first key tile
  const int nkt = min((N + C::BT - 1) / C::BT - kt0, tps);  // tiles of the range
  load_tile(0, kt0);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  lds_barrier();
  for (int kt = 0; kt < nkt; ++kt) {  // kt counts the range's tiles
    const int st = kt & 1;
    if (kt + 1 < nkt) load_tile(st ^ 1, kt0 + kt + 1);
    const char *ks = Ks + st * C::TILEB, *vs = Vs + st * C::TILEB;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // S^T = K Q^T and dP^T = V dO^T: keys 32t + (8(r/4) + 4h + r%4), query l32 (keys
      // past N have zero K and V rows and add nothing to dQ)
      f32x16 s = {}, dp = {};
      const int kr = 32 * t + l32;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int off = kr * C::ROWB + (((2 * kc + h) ^ (kr & 15)) << 4);
        const f32x4 ka = *reinterpret_cast<const f32x4 *>(ks + off);
        const f32x4 va = *reinterpret_cast<const f32x4 *>(vs + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s = mma_f32(ka[i], qf[kc][i], s);
          dp = mma_f32(va[i], gf[kc][i], dp);
        }
      }
      // dQ^T += K^T dS^T, one key pair per step
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float ds = ex2(fmaf(s[r], c, -my_lse2)) * (dp[r] - my_d);
        const int key = 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int e = 0; e < OB; ++e)
          dq[e] = mma_f32(*reinterpret_cast<const float *>(ks + el_off32(key, 32 * e + l32, C::ROWB)),
                          ds, dq[e]);
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    lds_barrier();
  }

  constexpr int WAVE_LDS = (C::LDS / 4) & ~15;
  const int row0 = q0 + 32 * w;
  store_rows_lds<D, 1, false>(dq, 0.f, 1.f, 0.5f / scale, smem + w * WAVE_LDS,
                              dQ + slot + hoff + int64_t(row0) * D, nullptr, lane, N - row0);
}

// ------------------------------------------------------------------------------------
template <int D>
static hipError_t run_bwd32(const BwdProblem &p, float *dq, float *dk, float *dv, int nsplit,
                            int tps, hipStream_t stream) {
  using C = CfgB32<D>;
  const int64_t rows = int64_t(p.B) * p.H * p.N;
  {
    const int64_t blocks = (rows * (D / 4) + 255) / 256;
    const int grid = int(blocks < kMaxGrid ? blocks : kMaxGrid);
    hipLaunchKernelGGL((fa_bwd32_prep_kernel<D>), dim3(grid), dim3(256), 0, stream, p.o, p.dout,
                       p.lse, p.ws_lse2, p.ws_d, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const float c = p.scale * kLog2e;
  const int nb = (p.N + C::BR - 1) / C::BR;
  const int G = nb * p.B * p.H * nsplit;
  const float *q = static_cast<const float *>(p.q), *k = static_cast<const float *>(p.k),
              *v = static_cast<const float *>(p.v);
  {
    auto kern = fa_bwd32_dkdv_kernel<D>;
    const hipError_t ea = allow_lds_on_device<fa_bwd32_dkdv_kernel<D>>(C::LDS);
    if (ea != hipSuccess) return ea;
    hipLaunchKernelGGL(kern, dim3(G), dim3(C::NT), C::LDS, stream, q, k, v, p.dout, p.ws_lse2,
                       p.ws_d, dk, dv, p.N, nb, G, c, p.scale, nsplit, tps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    auto kern = fa_bwd32_dq_kernel<D>;
    const hipError_t ea = allow_lds_on_device<fa_bwd32_dq_kernel<D>>(C::LDS);
    if (ea != hipSuccess) return ea;
    hipLaunchKernelGGL(kern, dim3(G), dim3(C::NT), C::LDS, stream, q, k, v, p.dout, p.ws_lse2,
                       p.ws_d, dq, p.N, nb, G, c, p.scale, nsplit, tps);
  }
  return hipGetLastError();
}

hipError_t launch_bwd32_ranges(const BwdProblem &p, float *dq, float *dk, float *dv, int nsplit,
                               int tps, hipStream_t stream) {
  return p.d == 128 ? run_bwd32<128>(p, dq, dk, dv, nsplit, tps, stream)
                    : run_bwd32<64>(p, dq, dk, dv, nsplit, tps, stream);
}

hipError_t launch_bwd32(const BwdProblem &p, hipStream_t stream) {
  return launch_bwd32_ranges(p, p.dq, p.dk, p.dv, 1, (p.N + 63) / 64, stream);
}

}  // namespace fa
