// Fused attention forward for gfx950 (FlashAttention forward pass).
//
// Algorithm: MUSA SDK guide "FlashAttention optimization", FlashAttention formula
// steps 1-4 / a-f, with the FlashAttention-2 split of the grid over Q blocks
// (same guide, "FlashAttention-2 improvement") and the Q-resident, K/V-streaming
// loop order of the pwwt.cn CK/MI50 notes (section 2.2).  Per workgroup:
//
//   prologue  Q tile [BM x d] -> LDS with coalesced 16-byte loads -> registers
//   loop      K_j, V_j tiles stream through two LDS stages; while tile j is used,
//             tile j+1 is already in flight from global memory
//             S^T = K_j Q^T on the matrix cores (fp32 accumulate)
//             online softmax in registers: m_new = max(m, rowmax S),
//             alpha = 2^(c m - c m_new), P = 2^(c S - c m_new), l = alpha l + rowsum P,
//             with c = scale * log2(e) folded into one multiply-add per score
//             O = alpha O (rescaled BEFORE the new block is added), then
//             O^T += V_j^T P^T on the matrix cores
//   epilogue  O / l and LSE = m*scale + ln l to global memory
//
// This unit holds the fp32-input kernel, the merge of key ranges and the dispatch (the
// 16-bit kernel is fa_fwd16.hpp).  Layout of the fp32 kernel's work on the chip: 4 waves
// x 32 query rows.  Each wave computes S^T so that every lane owns ONE query row and 16
// (of 32) keys per 32x32 block: the row
// max and row sum are in-lane reductions plus one exchange with lane ^ 32, and the
// rescale factor alpha is a per-lane scalar.  The P registers feed the P V product
// directly; V stays row-major in LDS and its operand is fetched with the
// transposing LDS load in the same key order the P registers hold.
#include "fa_internal.h"
#include "fa_softmax.hpp"

namespace fa {

// ====================================================================================
// fp32 inputs, d in {64, 128, 256}: fp32 matrix cores, fp32 P
// ====================================================================================
template <int D>
struct Cfg32 {
  static constexpr int BM = kFusedBM;
  static constexpr int BN = D == 256 ? 32 : 64;  // two K and two V stages fit in LDS
  static constexpr int ROWB = D * 4;
  static constexpr int CPR = ROWB / 16;
  static constexpr int TILEB = BN * ROWB;
  static constexpr int CPT = TILEB / 16 / 256;
  static constexpr int QCPT = BM * CPR / 256;
  static constexpr int SB = BN / 32;
  static constexpr int KC = D / 8;  // 16-byte chunks per lane half: 4 k-steps each
  static constexpr int OB = D / 32;
  static constexpr int LDS = 4 * TILEB;
  static_assert(BM * ROWB <= LDS, "Q staging must fit in the K and V stages");
  // at d = 256, Q and O fill the registers: fence the unrolled loops so that the LDS
  // operand reads are not hoisted far ahead of their products
  static constexpr bool FENCE = D == 256;
};

// STATS: the statistics-recording form (nsplit = 1): after every key tile each query
// row's running max (base-2 units) and row sum go to ST, as in fa_fwd16_kernel.
template <int D, bool STATS = false>
__global__ __launch_bounds__(256, 1) void fa_fwd32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, int N, int nqt, int G, float c, int nsplit,
    int kps, float *__restrict__ ST) {
  using C = Cfg32<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char *const Ks = smem;
  char *const Vs = smem + 2 * C::TILEB;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  // work decomposition and key ranges as in fa_fwd16_kernel (nsplit = 1: whole head)
  const int L = xcd_remap(blockIdx.x, G);
  const int qt = L % nqt, kg = (L / nqt) % nsplit, bh = L / nqt / nsplit;
  const int q0 = qt * C::BM;
  const int64_t hoff = int64_t(bh) * N * D;
  const int64_t bhn = int64_t(G / (nqt * nsplit)) * N;
  const int kbeg = kg * kps, NK = min(N - kbeg, kps);
  const float *Qh = Q + hoff, *Kh = K + hoff + int64_t(kbeg) * D, *Vh = V + hoff + int64_t(kbeg) * D;

#pragma unroll
  for (int i = 0; i < C::QCPT; ++i) {
    const int cid = i * 256 + tid, r = cid / C::CPR, ch = cid % C::CPR;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (q0 + r < N) val = *reinterpret_cast<const u32x4 *>(Qh + int64_t(q0 + r) * D + ch * 4);
    lds_write16(Ks, r * C::ROWB + swz_row<C::CPR>(r, ch) * 16, val);
  }
  __syncthreads();
  // k-step 4*kc + i of the Q K product uses column 8kc + 4h + i on both operands
  f32x4 qf[C::KC];
  {
    const int qr = 32 * w + l32;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc)
      qf[kc] = __builtin_bit_cast(
          f32x4, lds_read16(Ks, qr * C::ROWB + swz_row<C::CPR>(qr, 2 * kc + h) * 16));
  }
  __syncthreads();

  u32x4 kreg[C::CPT], vreg[C::CPT];
  auto fetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int cid = i * 256 + tid, r = cid / C::CPR, ch = cid % C::CPR;
      const int key = kt * C::BN + r;
      kreg[i] = vreg[i] = u32x4{0u, 0u, 0u, 0u};
      if (key < NK) {
        kreg[i] = *reinterpret_cast<const u32x4 *>(Kh + int64_t(key) * D + ch * 4);
        vreg[i] = *reinterpret_cast<const u32x4 *>(Vh + int64_t(key) * D + ch * 4);
      }
    }
  };
  auto stage = [&](int buf) {
    char *kb = Ks + buf * C::TILEB, *vb = Vs + buf * C::TILEB;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int cid = i * 256 + tid, r = cid / C::CPR, ch = cid % C::CPR;
      lds_write16(kb, r * C::ROWB + swz_row<C::CPR>(r, ch) * 16, kreg[i]);
      lds_write16(vb, r * C::ROWB + swz_row<C::CPR>(r, ch) * 16, vreg[i]);
    }
  };

  f32x16 o[C::OB];
#pragma unroll
  for (int e = 0; e < C::OB; ++e) o[e] = f32x16{};
  float mc = -INFINITY, l = 0.f;

  // the next tile's loads are issued before the current tile's compute; at d = 256 the
  // registers that would hold them in flight are not there, so they follow it
  constexpr bool PREFETCH = D <= 128;
  const int nkt = (NK + C::BN - 1) / C::BN;
  fetch(0);
  stage(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const char *kb = Ks + buf * C::TILEB;
    const char *vb = Vs + buf * C::TILEB;
    if (PREFETCH && kt + 1 < nkt) fetch(kt + 1);

    // at d = 256, lane ids re-pinned per tile keep the operand offsets computed next to
    // their use instead of hoisted out of the loop into registers
    int lx = l32, hx = h;
    if constexpr (C::FENCE) {
      pin(lx);
      pin(hx);
    }
    f32x16 s[C::SB];
#pragma unroll
    for (int t = 0; t < C::SB; ++t) {
      s[t] = f32x16{};
      const int kr = 32 * t + lx;
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) {
        f32x4 kf = __builtin_bit_cast(
            f32x4, lds_read16(kb, kr * C::ROWB + swz_row<C::CPR>(kr, 2 * kc + hx) * 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) s[t] = mma_f32(kf[i], qf[kc][i], s[t]);
        if constexpr (C::FENCE) __builtin_amdgcn_sched_barrier(0);
      }
    }

    const int nvalid = NK - kt * C::BN;
    if (nvalid < C::BN)
      softmax_tile<C::SB, C::OB, true>(s, o, mc, l, c, nvalid, h);
    else
      softmax_tile<C::SB, C::OB, false>(s, o, mc, l, c, nvalid, h);
    if constexpr (STATS) {
      // a tile of 32 keys at d = 256: the record is per 64 keys, after every second tile
      constexpr int TPR = 64 / C::BN;  // tiles per record
      const float lt = pair_sum(l);
      const int row = q0 + 32 * w + l32;
      if ((kt % TPR == TPR - 1 || kt == nkt - 1) && h == 0 && row < N) {
        const int ntr = (NK + 63) / 64;
        float *p = ST + ((int64_t(bh) * N + row) * ntr + kt / TPR) * 2;
        p[0] = mc;
        p[1] = lt;
      }
    }

    // O^T += V^T P^T, one key pair per step: register r of block t holds, on lane half
    // h, key 32t + 8(r/4) + 4h + r%4; the V operand is that key's row, column 32e + l32
#pragma unroll
    for (int e = 0; e < C::OB; ++e) {
      const int col = 32 * e + lx, ch = col >> 2, cb = (col & 3) * 4;
#pragma unroll
      for (int t = 0; t < C::SB; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * t + 8 * (r >> 2) + 4 * hx + (r & 3);
          const float vv =
              *reinterpret_cast<const float *>(vb + key * C::ROWB + swz_row<C::CPR>(key, ch) * 16 + cb);
          o[e] = mma_f32(vv, s[t][r], o[e]);
          if constexpr (C::FENCE)
            if (r % 4 == 3) __builtin_amdgcn_sched_barrier(0);
        }
    }

    if (kt + 1 < nkt) {
      if (!PREFETCH) fetch(kt + 1);
      stage(buf ^ 1);
    }
    __syncthreads();
  }

  const int row = q0 + 32 * w + l32;
  store_rows<C::OB>(o, mc, l, l, O + kg * bhn * D + hoff + int64_t(row) * D,
                    LSE + kg * bhn + int64_t(bh) * N + row, h,
                    row < N);
}

// ------------------------------------------------------------------------------------

template <int D, bool STATS = false>
static hipError_t run32(const Problem &p, float *o, float *lse, int nsplit, int kps,
                        hipStream_t stream, float *stats = nullptr) {
  using C = Cfg32<D>;
  auto kern = fa_fwd32_kernel<D, STATS>;
  const hipError_t ea = allow_lds_on_device<fa_fwd32_kernel<D, STATS>>(C::LDS);
  if (ea != hipSuccess) return ea;
  const int nqt = (p.N + C::BM - 1) / C::BM;
  const int G = nqt * p.B * p.H * nsplit;
  const float c = p.scale * kLog2e;
  hipLaunchKernelGGL(kern, dim3(G), dim3(256), C::LDS, stream,
                     static_cast<const float *>(p.q), static_cast<const float *>(p.k),
                     static_cast<const float *>(p.v), o, lse, p.N, nqt, G, c, nsplit, kps,
                     stats);
  return hipGetLastError();
}

static hipError_t run32_any(const Problem &p, float *o, float *lse, int nsplit, int kps,
                            hipStream_t stream) {
  return p.d == 256 ? run32<256>(p, o, lse, nsplit, kps, stream)
         : p.d == 128 ? run32<128>(p, o, lse, nsplit, kps, stream)
                      : run32<64>(p, o, lse, nsplit, kps, stream);
}

hipError_t launch_fused(const Problem &p, hipStream_t stream) {
  switch (p.dtype) {
    case kF16:
    case kBF16:
      return launch_fwd16(p, p.o, p.lse, 1, p.N, stream);
    default:
      return run32_any(p, p.o, p.lse, 1, p.N, stream);
  }
}

hipError_t launch_fused_stats(const Problem &p, float *stats, hipStream_t stream) {
  if (p.dtype != kF32) return launch_fwd16(p, p.o, p.lse, 1, p.N, stream, stats);
  return p.d == 256 ? run32<256, true>(p, p.o, p.lse, 1, p.N, stream, stats)
         : p.d == 128 ? run32<128, true>(p, p.o, p.lse, 1, p.N, stream, stats)
                      : run32<64, true>(p, p.o, p.lse, 1, p.N, stream, stats);
}

// ------------------------------------------------------------------------------------
// Key-split forward.  The keys of every head are cut into ranges of kps keys; one
// launch of the fused kernel computes, for each range g, the attention of every query
// row over that range alone (O_g, normalised by its own row sum, and LSE_g), and the
// merge kernel combines the ranges with the block-merge rule of the Triton tutorial
// (section 2.3) and the MUSA guide's block update (step e):
//   LSE = log sum_g exp(LSE_g),   O = sum_g exp(LSE_g - LSE) O_g,
// evaluated against M = max_g LSE_g for range safety.  Rows are independent; each
// thread owns 4 columns of one row.
template <int D>
__global__ __launch_bounds__(256) void fa_merge_kernel(const float *__restrict__ Opart,
                                                       const float *__restrict__ Lpart,
                                                       float *__restrict__ O,
                                                       float *__restrict__ LSE, int64_t rows,
                                                       int nsplit) {
  constexpr int TPR = D / 4;      // threads per row
  constexpr int RPB = 256 / TPR;  // rows per workgroup
  const int64_t row = int64_t(blockIdx.x) * RPB + threadIdx.x / TPR;
  const int col = 4 * (threadIdx.x % TPR);
  if (row >= rows) return;
  float m = -INFINITY;
  for (int g = 0; g < nsplit; ++g) m = fmaxf(m, Lpart[g * rows + row]);
  float wsum = 0.f, a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int g = 0; g < nsplit; ++g) {
    const float wg = expf(Lpart[g * rows + row] - m);
    const f32x4 v = *reinterpret_cast<const f32x4 *>(Opart + (g * rows + row) * D + col);
    wsum += wg;
    a0 = fmaf(wg, v[0], a0);
    a1 = fmaf(wg, v[1], a1);
    a2 = fmaf(wg, v[2], a2);
    a3 = fmaf(wg, v[3], a3);
  }
  const float inv = 1.0f / wsum;
  *reinterpret_cast<f32x4 *>(O + row * D + col) = f32x4{a0 * inv, a1 * inv, a2 * inv, a3 * inv};
  if (col == 0) LSE[row] = m + logf(wsum);
}

template <int D>
static hipError_t run_merge(const Problem &p, const float *opart, const float *lpart,
                            int nsplit, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 4);
  const int64_t rows = int64_t(p.B) * p.H * p.N;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL(fa_merge_kernel<D>, dim3(unsigned(blocks)), dim3(256), 0, stream, opart,
                     lpart, p.o, p.lse, rows, nsplit);
  return hipGetLastError();
}

hipError_t launch_fused_split(const Problem &p, float *opart, float *lpart, int nsplit,
                              int kps, hipStream_t stream) {
  hipError_t e = p.dtype == kF32 ? run32_any(p, opart, lpart, nsplit, kps, stream)
                                 : launch_fwd16(p, opart, lpart, nsplit, kps, stream);
  if (e != hipSuccess) return e;
  return p.d == 256 ? run_merge<256>(p, opart, lpart, nsplit, stream)
         : p.d == 128 ? run_merge<128>(p, opart, lpart, nsplit, stream)
                      : run_merge<64>(p, opart, lpart, nsplit, stream);
}

}  // namespace fa
