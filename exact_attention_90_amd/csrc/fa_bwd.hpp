// Attention backward pass for gfx950: dQ, dK and dV of O = softmax(scale Q K^T) V.
//
// Method (pwwt.cn Triton tutorial, sections 2.4 and 4.4): P is never stored; the
// backward pass recomputes it from the inputs and the forward pass's row statistic
// (LSE = m + ln l), then applies the chain rule:
//
//   P   = exp(scale S - LSE)              S = Q K^T, recomputed tile by tile
//   dV  = P^T dO
//   dP  = dO V^T
//   D_i = <dO_i, O_i>                     (= sum_j P_ij dP_ij, the softmax Jacobian's
//                                          row term, from the stored output)
//   dS  = P * (dP - D)
//   dQ  = scale dS K,   dK = scale dS^T Q
//
// Three kernels, every contraction on the matrix cores (v_mfma_f32_32x32x16 in the input
// type with fp32 accumulation; P and dS are rounded to the input type for theirs):
//   prep   D_i, LSE_i log2(e), and dO rounded to the input type (one pass over O, dO)
//   dkdv   one workgroup per 32W keys of a head, each wave owning 32 keys: its K and V
//          rows stay in registers while Q and dO tiles stream through LDS; dK and dV
//          accumulate in registers (the lane owns a key, like the query in the forward)
//   dq     one workgroup per 32W queries: its Q and dO rows stay in registers while K
//          and V tiles stream through LDS; dQ accumulates in registers
// No atomics: every output element is written once, so results are deterministic.
#pragma once

#include <type_traits>

#include "fa_internal.h"
#include "fa_softmax.hpp"

namespace fa {

// LDS reads from an absolute 32-bit LDS byte address (lds_addr, lds_read16_at and
// lds_read_tr_at in fa_device.hpp)
__device__ __forceinline__ f32x4 lds_read_f32x4_at(uint32_t addr) {
  return __builtin_bit_cast(f32x4, *(const lds_u32x4 *)(uintptr_t)addr);
}

// A streamed tile is read two ways: 16-byte row reads (the A operand of S = Q K^T and
// dP = dO V^T) and transposing reads (the A operand of dV^T = dO^T P and dK^T = Q^T dS,
// or of dQ^T = K^T dS^T).  One XOR key per row serves both without bank conflicts: over
// any 16 consecutive rows it is a bijection (the row reads), and its bits that select
// the 64-byte block differ across 4 consecutive rows (the transposing reads).
template <int CPR>
__device__ __forceinline__ int swz_both(int r) {
  if constexpr (CPR == 8)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else
    return ((r & 3) << 2) | ((r >> 2) & 3);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
template <bool BF16>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  if constexpr (BF16)
    return pack_bf16(a, b);
  else
    return pack_f16(a, b);
}
// the two 16-bit values of a packed word, widened exactly to fp32
template <bool BF16>
__device__ __forceinline__ void unpack16(uint32_t w, float &a, float &b) {
  if constexpr (BF16) {
    a = __builtin_bit_cast(float, w << 16);
    b = __builtin_bit_cast(float, w & 0xffff0000u);
  } else {
    const f16x2 v = __builtin_bit_cast(f16x2, w);
    a = (float)v[0];
    b = (float)v[1];
  }
}

// ------------------------------------------------------------------------------------
// prep: per row, D = <dO, O>, lse2 = LSE log2(e); dO rounded to the input type.  D takes
// dO as rounded for the dP product, so that sum_j P_ij dP_ij = D_i holds for the values
// the matrix cores multiply (up to the forward pass's own rounding in O).
// ------------------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_bwd_prep_kernel(const float *__restrict__ O,
                                                          const float *__restrict__ dO,
                                                          const float *__restrict__ LSE,
                                                          uint16_t *__restrict__ dO16,
                                                          float *__restrict__ lse2,
                                                          float *__restrict__ Dv, int64_t rows) {
  constexpr int TPR = D / 4;  // threads per row, 16 bytes of O and dO each
  const int64_t total = rows * TPR;
  for (int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x; gid - threadIdx.x < total;
       gid += int64_t(gridDim.x) * 256) {
    // every thread of a row runs the same iterations (rows never straddle a block)
    const int64_t row = gid / TPR;
    const int c = int(gid % TPR);
    float part = 0.f;
    if (row < rows) {
      const f32x4 o = *reinterpret_cast<const f32x4 *>(O + row * D + 4 * c);
      const f32x4 g = *reinterpret_cast<const f32x4 *>(dO + row * D + 4 * c);
      const u32x2 gw = {pack16<BF16>(g[0], g[1]), pack16<BF16>(g[2], g[3])};
      *reinterpret_cast<u32x2 *>(dO16 + row * D + 4 * c) = gw;
      float r0, r1, r2, r3;
      unpack16<BF16>(gw[0], r0, r1);
      unpack16<BF16>(gw[1], r2, r3);
      part = o[0] * r0 + o[1] * r1 + o[2] * r2 + o[3] * r3;
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (row < rows && c == 0) {
      Dv[row] = part;
      lse2[row] = LSE[row] * kLog2e;
    }
  }
}

// ------------------------------------------------------------------------------------
// shared configuration of the two main kernels
// ------------------------------------------------------------------------------------
template <int D, int WAVES>
struct CfgB {
  static constexpr int NT = 64 * WAVES;        // threads per workgroup
  static constexpr int BR = 32 * WAVES;        // resident rows (keys or queries) per workgroup
  static constexpr int BT = 64;                // rows per streamed tile
  static constexpr int ROWB = 2 * D;           // bytes per 16-bit row
  static constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  static constexpr int TILEB = BT * ROWB;      // bytes of one streamed tile
  static constexpr int CPT = TILEB / 16 / NT;  // chunks per thread per tile
  static constexpr int KC = D / 16;            // k-steps over d
  static constexpr int OB = D / 32;            // 32-column output blocks
  static constexpr int RSTEP = NT / CPR;       // rows between a thread's chunks
  // with 512-byte rows (d = 256) a thread's rows are 8 apart and their swizzle keys
  // alternate between two values
  static constexpr bool KFLIP = RSTEP % 16 != 0;
  static constexpr int STATB = 1024;           // one statistics stage (64 lanes x 16 B)
  static constexpr int LDS = 4 * TILEB + 4 * STATB;
  static_assert(CPT >= 1 && TILEB % (16 * NT) == 0, "a tile is whole chunks per thread");
  static_assert(RSTEP % 8 == 0, "a thread's rows alternate between at most two keys");
  static_assert(32 * D * 4 <= LDS / WAVES, "a wave's output rows fit its LDS share");
};

// Lane offsets into a streamed tile (bytes, without the stage offset):
//   row reads: row 32t + l32, logical chunk 2kc + h  ->  rb + 32t ROWB + ((32kc) ^ rx)
//   transposing reads for k-step u (rows 16u + 8x + ...), output block e:
//                                                     ->  tb[x] + 16u ROWB + ((64e) ^ tx)
template <int CPR, int ROWB>
struct TileLanes {
  int rb, rx, tb0, tb1, tx;
  __device__ __forceinline__ TileLanes(int lane) {
    const int h = lane >> 5, l32 = lane & 31;
    const int f = swz_both<CPR>(l32);  // rows 32t + l32 share the key of l32
    rb = l32 * ROWB + 16 * (h ^ (f & 1));
    rx = 32 * (f >> 1);
    // transposing read: lane j of 16-lane group G reads row 8x + 4(G/2) + j/4 (plus 16u)
    // at columns 32e + 16(G%2) + 4(j%4): chunk 4e + c0, byte (column % 8) * 2
    const int grp = lane >> 4, j16 = lane & 15;
    const int r0 = 4 * (grp >> 1) + (j16 >> 2);
    const int col = 16 * (grp & 1) + 4 * (j16 & 3);
    const int c0 = col >> 3, cb = (col & 7) * 2;
    const int f0 = swz_both<CPR>(r0), f1 = swz_both<CPR>(r0 + 8);
    // chunk (4e + c0) ^ f = 4 (e ^ (f >> 2)) + (c0 ^ (f & 3)); f >> 2 is the same for
    // rows r0 and r0 + 8
    tb0 = r0 * ROWB + 16 * (c0 ^ (f0 & 3)) + cb;
    tb1 = (r0 + 8) * ROWB + 16 * (c0 ^ (f1 & 3)) + cb;
    tx = 64 * (f0 >> 2);
  }
};

// ------------------------------------------------------------------------------------
// dkdv: dK and dV for the 32W keys of one workgroup.  WHAT selects the outputs
// (kDK | kDV): at d = 256 the rows of K, V, dK and dV of 32 keys exceed a SIMD's
// registers, so dV and dK are computed by two launches (each recomputes S).
// ------------------------------------------------------------------------------------
constexpr int kDK = 1, kDV = 2;
// minimum waves per SIMD the registers must allow (K, V, dK and dV rows of 32 keys take
// 6 d / 4 registers per lane)
template <int D>
constexpr int dkdv_wpe() { return D >= 128 ? 1 : 2; }
template <int D>
constexpr int dq_wpe() { return D >= 256 ? 1 : 2; }

template <int D, bool BF16, int WAVES, int WHAT>
__global__ __launch_bounds__(64 * WAVES, dkdv_wpe<D>()) void fa_bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO16,
    const float *__restrict__ lse2, const float *__restrict__ Dv, float *__restrict__ dK,
    float *__restrict__ dV, int N, int nkb, int G, float c, float scale, int nsplit, int tps) {
  using C = CfgB<D, WAVES>;
  constexpr int KC = C::KC, OB = C::OB, CPT = C::CPT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char *const Qs = smem;                    // Q tiles, two stages
  char *const Gs = smem + 2 * C::TILEB;     // dO tiles, two stages
  char *const Ls = smem + 4 * C::TILEB;     // lse2 of the tile's queries, two stages
  char *const Ds = Ls + 2 * C::STATB;       // D of the tile's queries, two stages

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // workgroup L: key block L % nkb, query range (L / nkb) % nsplit (query tiles
  // [rg tps, min(nqt, (rg + 1) tps)), never empty), head L / (nkb nsplit).  Its dK and dV
  // over that range go to slot rg of dK and dV (slots B H N d values apart); with
  // nsplit = 1 the range is every query and the slot is the gradient itself.
  const int L = xcd_remap(blockIdx.x, G);
  const int rg = (L / nkb) % nsplit, bh = L / nkb / nsplit, k0 = (L % nkb) * C::BR;
  const int64_t hoff = int64_t(bh) * N * D;
  const int64_t slot = int64_t(G / (nkb * nsplit)) * N * D * rg;
  const uint32_t head_bytes = uint32_t(N) * C::ROWB;
  const auto qrs = make_rsrc(Q + hoff, head_bytes);
  const auto grs = make_rsrc(dO16 + hoff, head_bytes);
  const auto krs = make_rsrc(K + hoff, head_bytes);
  const auto vrs = make_rsrc(V + hoff, head_bytes);
  const auto lrs = make_rsrc(lse2 + int64_t(bh) * N, uint32_t(N) * 4);
  const auto drs = make_rsrc(Dv + int64_t(bh) * N, uint32_t(N) * 4);

  // the wave's 32 keys: K and V rows as B operands (lane: key l32, columns 8h.. of each
  // 16-column k-step); keys past N read zeros
  constexpr bool WANT_DK = (WHAT & kDK) != 0, WANT_DV = (WHAT & kDV) != 0;
  // At d = 128, and for the dV-only launch at d = 256, the dV and dK products are written
  // as assembly accumulating in AGPRs, and the unit that instantiates the kernel
  // (fa_bwd_d128.hip, fa_bwd_d256.hip) is compiled with the compiler's own products (S,
  // dP) in vector-register form: S and dP are then never copied out of AGPRs (d = 128:
  // 128 moves per tile fewer, +5 %; d = 256, dV: +9 %; bitwise the same).  The dK-only
  // launch at d = 256 needs the AGPRs for S and dP (its vector registers are full).
  constexpr bool ASM_DKDV = D == 128 || (D == 256 && !WANT_DK);
  const int key = k0 + 32 * w + l32;
  u32x4 kf[KC], vf[WANT_DK ? KC : 1];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    kf[kc] = buf_load16(krs, key * C::ROWB + (2 * kc + h) * 16, 0);
    if constexpr (WANT_DK) vf[kc] = buf_load16(vrs, key * C::ROWB + (2 * kc + h) * 16, 0);
  }

  const TileLanes<C::CPR, C::ROWB> tl(lane);
  // loads of a tile into LDS: chunk i of thread tid is LDS chunk i NT + tid, i.e. row
  // i RSTEP + tid / CPR at physical chunk tid % CPR, which holds logical chunk
  // (tid % CPR) ^ key(row); every row of a thread has the same key
  const int srow = tid / C::CPR, sch = tid % C::CPR;
  const int st_off0 = srow * C::ROWB + (sch ^ swz_both<C::CPR>(srow)) * 16;
  const int st_off1 =
      C::KFLIP ? srow * C::ROWB + (sch ^ swz_both<C::CPR>(srow + C::RSTEP)) * 16 : st_off0;
  auto st_off = [&](int i) { return (C::KFLIP && (i & 1)) ? st_off1 : st_off0; };
  constexpr int ST_STEP = C::NT * 16;
  const int dma_wave = wu * 1024;
  auto load_chunk = [&](int stage, int qt, int i) {
    buf_load16_lds(qrs, Qs + stage * C::TILEB + dma_wave + i * ST_STEP, st_off(i),
                   qt * C::TILEB + i * ST_STEP);
    buf_load16_lds(grs, Gs + stage * C::TILEB + dma_wave + i * ST_STEP, st_off(i),
                   qt * C::TILEB + i * ST_STEP);
  };
  auto load_stats = [&](int stage, int qt) {
    // the tile's 64 values of lse2 and D (lanes 16..63 bring bytes no one reads)
    if (wu == 0) buf_load16_lds(lrs, Ls + stage * C::STATB, lane * 16, qt * 256);
    if (WANT_DK && wu == WAVES - 1)
      buf_load16_lds(drs, Ds + stage * C::STATB, lane * 16, qt * 256);
  };
  auto load_tile = [&](int stage, int qt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) load_chunk(stage, qt, i);
    load_stats(stage, qt);
  };
  // at d >= 128 the next tile's loads ride one per step between the A0 matrix-core steps
  // instead of all issuing before them
  static_assert(D < 128 || CPT < C::KC, "one load per A0 step");

  f32x16 dk[WANT_DK ? OB : 1], dv[WANT_DV ? OB : 1];
#pragma unroll
  for (int e = 0; e < OB; ++e) {
    if constexpr (WANT_DK) dk[e] = f32x16{};
    if constexpr (WANT_DV) dv[e] = f32x16{};
  }

  const int qt0 = rg * tps;                                       // first query tile
  const int nqt = min((N + C::BT - 1) / C::BT - qt0, tps);         // tiles of the range
  // LDS addresses of the operand reads in the current stage, one per k-step (row reads)
  // and per output block (transposing reads); the dO tiles are an immediate offset from
  // them.  The stages are TILEB (statistics: STATB) apart, so one add per register moves
  // them to the next tile's stage.
  const uint32_t q_lds = lds_addr(Qs);
  uint32_t a_off[KC], b_off0[OB], b_off1[OB];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) a_off[kc] = q_lds + (tl.rb + ((32 * kc) ^ tl.rx));
#pragma unroll
  for (int e = 0; e < OB; ++e) {
    b_off0[e] = q_lds + (tl.tb0 + ((64 * e) ^ tl.tx));
    b_off1[e] = q_lds + (tl.tb1 + ((64 * e) ^ tl.tx));
  }
  // statistics of queries 4h + (8g + 32t): this lane's 16-byte group, stage 0
  uint32_t stat_off = q_lds + 4 * C::TILEB + 16 * h;
  constexpr int GS = 2 * C::TILEB;   // dO tile stage - Q tile stage
  constexpr int DS = 2 * C::STATB;   // D stage - lse2 stage
  load_tile(0, qt0);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  lds_barrier();
  for (int qt = 0; qt < nqt; ++qt) {  // qt counts the range's tiles
    const int st = qt & 1;
    // the other stage held tile qt - 1, released by the barrier that ended it
    const bool more = qt + 1 < nqt;
    if (D < 128 && more) load_tile(st ^ 1, qt0 + qt + 1);
    // held in registers across the loop rather than recomputed at each read
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) pin(a_off[kc]);
#pragma unroll
    for (int e = 0; e < OB; ++e) {
      pin(b_off0[e]);
      pin(b_off1[e]);
    }
    pin(stat_off);
    if constexpr (D >= 128) {
      // The tile's two 32-query blocks t = 0, 1 go through three parts:
      //   A(t)  S = Q K^T and dP = dO V^T for queries 32t + (8(r/4) + 4h + r%4), key l32
      //         (matrix cores; the tiles read as rows)
      //   V(t)  P = 2^(c s - lse2_q), dS = P (dP - D_q), both packed into the operand
      //         layout of B (VALU)
      //   B(t)  dV^T += dO^T P and dK^T += Q^T dS (matrix cores; the tiles read transposed)
      // in four phases, A0 | A1 + V0 | B0 + V1 | B1, so that the vector work of one block
      // rides between the matrix-core steps of the other.  Operand reads run PA (A) and
      // PB (B) steps ahead, in rings indexed by the step's position in the tile (block t,
      // step kc is position t KC + kc), so that the next block's first reads never take a
      // slot this block still needs; fences keep every step in place.
      {
        constexpr int PA = 4, PB = 2, NB = 2 * OB;
        static_assert(PA <= KC && PB <= NB, "prefetch depth within one part");
        f32x16 s[2], dp[2];
        float p[2][16], ds[2][16];
        u32x4 pf[2][2], sf[2][2];
        f32x4 lq[2][4], dq4[2][4];
        u32x4 qa[PA], ga[PA], bg[PB], bq[PB];
        // A operands: rows 32t + l32 of the Q and dO tiles at logical chunk 2kc + h
        auto a_load = [&](int t, int kc) {
          const uint32_t off = a_off[kc] + 32 * t * C::ROWB;
          const int slot = (t * KC + kc) % PA;
          qa[slot] = lds_read16_at(off);
          if constexpr (WANT_DK) ga[slot] = lds_read16_at(off + GS);
        };
        auto a_step = [&](int t, int kc) {
          const int slot = (t * KC + kc) % PA;
          s[t] = mma16<BF16>(qa[slot], kf[kc], kc == 0 ? f32x16{} : s[t]);
          if constexpr (WANT_DK) dp[t] = mma16<BF16>(ga[slot], vf[kc], kc == 0 ? f32x16{} : dp[t]);
        };
        // statistics of the 16 queries block t's registers hold: 32t + 8g + 4h + 0..3
        auto stat_load = [&](int t) {
  #pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint32_t qo = stat_off + (32 * t + 8 * g) * 4;
            lq[t][g] = lds_read_f32x4_at(qo);
            if constexpr (WANT_DK) dq4[t][g] = lds_read_f32x4_at(qo + DS);
          }
        };
        // V(t) for registers lo .. hi-1; operand block x (registers 8x .. 8x + 7: queries
        // 16(2t + x) + 8y + 4h + s4 in slot 4y + s4) is packed once its 8 values exist
        auto v_range = [&](int t, int lo, int hi) {
  #pragma unroll
          for (int r = 0; r < 16; ++r)
            if (r >= lo && r < hi) {
              // taken into vector registers at this step (left alone, the compiler moves
              // the whole block's vector work up to where its products end, where no
              // matrix-core step runs beside it)
              float sv = s[t][r], gv = WANT_DK ? dp[t][r] : 0.f;
              pin(sv);
              if constexpr (WANT_DK) pin(gv);
              p[t][r] = ex2(fmaf(sv, c, -lq[t][r >> 2][r & 3]));
              ds[t][r] = WANT_DK ? p[t][r] * (gv - dq4[t][r >> 2][r & 3]) : 0.f;
            }
  #pragma unroll
          for (int x = 0; x < 2; ++x)
            if (hi >= 8 * x + 8 && lo < 8 * x + 8) {
              const float *a = p[t] + 8 * x, *b = ds[t] + 8 * x;
              pf[t][x] = u32x4{pack16<BF16>(a[0], a[1]), pack16<BF16>(a[2], a[3]),
                               pack16<BF16>(a[4], a[5]), pack16<BF16>(a[6], a[7])};
              if constexpr (WANT_DK)
                sf[t][x] = u32x4{pack16<BF16>(b[0], b[1]), pack16<BF16>(b[2], b[3]),
                                 pack16<BF16>(b[4], b[5]), pack16<BF16>(b[6], b[7])};
            }
        };
        // B step i of block t: k-step u = 2t + i / OB (16 queries), output block e = i % OB
        auto b_load = [&](int t, int i) {
          const int u = 2 * t + i / OB, e = i % OB;
          const uint32_t o0 = b_off0[e] + 16 * u * C::ROWB;
          const uint32_t o1 = b_off1[e] + 16 * u * C::ROWB;
          const int slot = (t * NB + i) % PB;
          if constexpr (WANT_DV) {
            const u32x2 g0 = lds_read_tr_at(o0 + GS), g1 = lds_read_tr_at(o1 + GS);
            bg[slot] = u32x4{g0[0], g0[1], g1[0], g1[1]};
          }
          if constexpr (WANT_DK) {
            const u32x2 q0 = lds_read_tr_at(o0), q1 = lds_read_tr_at(o1);
            bq[slot] = u32x4{q0[0], q0[1], q1[0], q1[1]};
          }
        };
        auto b_step = [&](int t, int i) {
          const int x = i / OB, e = i % OB, slot = (t * NB + i) % PB;
          if constexpr (ASM_DKDV) {
            if constexpr (BF16) {
              if constexpr (WANT_DV)
                asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                             : "+a"(dv[e]) : "v"(bg[slot]), "v"(pf[t][x]));
              if constexpr (WANT_DK)
                asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                             : "+a"(dk[e]) : "v"(bq[slot]), "v"(sf[t][x]));
            } else {
              if constexpr (WANT_DV)
                asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                             : "+a"(dv[e]) : "v"(bg[slot]), "v"(pf[t][x]));
              if constexpr (WANT_DK)
                asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                             : "+a"(dk[e]) : "v"(bq[slot]), "v"(sf[t][x]));
            }
          } else {
            if constexpr (WANT_DV) dv[e] = mma16<BF16>(bg[slot], pf[t][x], dv[e]);
            if constexpr (WANT_DK) dk[e] = mma16<BF16>(bq[slot], sf[t][x], dk[e]);
          }
        };

        stat_load(0);
  #pragma unroll
        for (int kc = 0; kc < PA; ++kc) a_load(0, kc);
        __builtin_amdgcn_sched_barrier(0);
        // A0
  #pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          a_step(0, kc);
          if (kc + PA < KC) a_load(0, kc + PA);
          else a_load(1, kc + PA - KC);
          if (more && kc < CPT) load_chunk(st ^ 1, qt0 + qt + 1, kc);
          if (more && kc == CPT) load_stats(st ^ 1, qt0 + qt + 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        stat_load(1);
        // A1 + V0
  #pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          a_step(1, kc);
          if (kc + PA < KC) a_load(1, kc + PA);
          else if (kc + PA - KC < PB) b_load(0, kc + PA - KC);
          v_range(0, kc * 16 / KC, (kc + 1) * 16 / KC);
          __builtin_amdgcn_sched_barrier(0);
        }
        // the B operands PA .. PB - 1 of block 0 that A1 had no step left to carry
  #pragma unroll
        for (int i = (PA < PB ? PA : PB); i < PB; ++i) b_load(0, i);
        // B0 + V1
  #pragma unroll
        for (int i = 0; i < NB; ++i) {
          b_step(0, i);
          if (i + PB < NB) b_load(0, i + PB);
          else b_load(1, i + PB - NB);
          v_range(1, i * 16 / NB, (i + 1) * 16 / NB);
          __builtin_amdgcn_sched_barrier(0);
        }
        // B1
  #pragma unroll
        for (int i = 0; i < NB; ++i) {
          b_step(1, i);
          if (i + PB < NB) b_load(1, i + PB);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      // d = 64: the simple order (the pipelined one needs more registers than three waves
      // per SIMD leave, and runs slower there)
  #pragma unroll
      for (int t = 0; t < 2; ++t) {  // 32-query blocks of the tile
        // S = Q K^T and dP = dO V^T for queries 32t + (8(r/4) + 4h + r%4), key l32
        f32x16 s = {}, dp = {};
  #pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const uint32_t off = a_off[kc] + 32 * t * C::ROWB;
          s = mma16<BF16>(lds_read16_at(off), kf[kc], s);
          if constexpr (WANT_DK) dp = mma16<BF16>(lds_read16_at(off + GS), vf[kc], dp);
        }
        // P = 2^(c s - lse2_q), dS = P (dP - D_q); the statistics of queries
        // 32t + 8g + 4h + 0..3 are one 16-byte broadcast read each
        float p[16], ds[16];
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t qo = stat_off + (32 * t + 8 * g) * 4;
          const f32x4 l4 = lds_read_f32x4_at(qo);
          f32x4 d4 = {};
          if constexpr (WANT_DK) d4 = lds_read_f32x4_at(qo + DS);
  #pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            const int r = 4 * g + s4;
            p[r] = ex2(fmaf(s[r], c, -l4[s4]));
            ds[r] = WANT_DK ? p[r] * (dp[r] - d4[s4]) : 0.f;
          }
        }
        // operands of k-steps 2t, 2t + 1: registers 8x .. 8x + 7 hold queries
        // 16(2t + x) + 8y + 4h + s4 in slot 4y + s4
  #pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int rb = 8 * x;
          const u32x4 pf = {pack16<BF16>(p[rb + 0], p[rb + 1]), pack16<BF16>(p[rb + 2], p[rb + 3]),
                            pack16<BF16>(p[rb + 4], p[rb + 5]), pack16<BF16>(p[rb + 6], p[rb + 7])};
          const u32x4 sf = {pack16<BF16>(ds[rb + 0], ds[rb + 1]), pack16<BF16>(ds[rb + 2], ds[rb + 3]),
                            pack16<BF16>(ds[rb + 4], ds[rb + 5]), pack16<BF16>(ds[rb + 6], ds[rb + 7])};
          const int u = 2 * t + x;
  #pragma unroll
          for (int e = 0; e < OB; ++e) {
            const uint32_t o0 = b_off0[e] + 16 * u * C::ROWB;
            const uint32_t o1 = b_off1[e] + 16 * u * C::ROWB;
            if constexpr (WANT_DV) {
              const u32x2 g0 = lds_read_tr_at(o0 + GS), g1 = lds_read_tr_at(o1 + GS);
              dv[e] = mma16<BF16>(u32x4{g0[0], g0[1], g1[0], g1[1]}, pf, dv[e]);
            }
            if constexpr (WANT_DK) {
              const u32x2 q0 = lds_read_tr_at(o0), q1 = lds_read_tr_at(o1);
              dk[e] = mma16<BF16>(u32x4{q0[0], q0[1], q1[0], q1[1]}, sf, dk[e]);
            }
          }
        }
      }
    }
    const int flip = st ? -C::TILEB : C::TILEB;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) a_off[kc] += flip;
#pragma unroll
    for (int e = 0; e < OB; ++e) {
      b_off0[e] += flip;
      b_off1[e] += flip;
    }
    stat_off += st ? -C::STATB : C::STATB;
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));  // tile qt + 1 has landed
    lds_barrier();
  }

  if constexpr (ASM_DKDV) {
    // the assembly products' results: wait for the last, then give dK and dV fresh
    // definitions, so that every read of them below follows the wait
    mfma_drain();
#pragma unroll
    for (int e = 0; e < OB; ++e) {
      if constexpr (WANT_DK) asm volatile("" : "+a"(dk[e]));
      if constexpr (WANT_DV) asm volatile("" : "+a"(dv[e]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // dK = scale dK^T (the lane's key column), dV; each through the wave's LDS share
  constexpr int WAVE_LDS = (C::LDS / WAVES) & ~15;
  const int row0 = k0 + 32 * w;
  char *region = smem + w * WAVE_LDS;
  // store_rows_lds divides by the pair sum of its normaliser: 1/scale for dK, 1 for dV
  if constexpr (WANT_DK)
    store_rows_lds<D, 1, false>(dk, 0.f, 1.f, 0.5f / scale, region,
                                dK + slot + hoff + int64_t(row0) * D, nullptr, lane, N - row0);
  if constexpr (WANT_DV)
    store_rows_lds<D, 1, false>(dv, 0.f, 1.f, 0.5f, region,
                                dV + slot + hoff + int64_t(row0) * D, nullptr, lane, N - row0);
}

// ------------------------------------------------------------------------------------
// dq: dQ for the 32W queries of one workgroup
// ------------------------------------------------------------------------------------
template <int D, bool BF16, int WAVES>
__global__ __launch_bounds__(64 * WAVES, dq_wpe<D>()) void fa_bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO16,
    const float *__restrict__ lse2, const float *__restrict__ Dv, float *__restrict__ dQ, int N,
    int nqb, int G, float c, float scale, int nsplit, int tps) {
  using C = CfgB<D, WAVES>;
  constexpr int KC = C::KC, OB = C::OB, CPT = C::CPT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char *const Ks = smem;                 // K tiles, two stages
  char *const Vs = smem + 2 * C::TILEB;  // V tiles, two stages

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // workgroup L: query block L % nqb, key range (L / nqb) % nsplit (key tiles
  // [rg tps, min(nkt, (rg + 1) tps))), head L / (nqb nsplit); its dQ over that range goes
  // to slot rg of dQ, as in the dK/dV kernel
  const int L = xcd_remap(blockIdx.x, G);
  const int rg = (L / nqb) % nsplit, bh = L / nqb / nsplit, q0 = (L % nqb) * C::BR;
  const int64_t hoff = int64_t(bh) * N * D;
  const int64_t slot = int64_t(G / (nqb * nsplit)) * N * D * rg;
  const uint32_t head_bytes = uint32_t(N) * C::ROWB;
  const auto qrs = make_rsrc(Q + hoff, head_bytes);
  const auto grs = make_rsrc(dO16 + hoff, head_bytes);
  const auto krs = make_rsrc(K + hoff, head_bytes);
  const auto vrs = make_rsrc(V + hoff, head_bytes);

  // the wave's 32 queries: Q and dO rows as B operands, and the row statistics
  const int row = q0 + 32 * w + l32;
  u32x4 qf[KC], gf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    qf[kc] = buf_load16(qrs, row * C::ROWB + (2 * kc + h) * 16, 0);
    gf[kc] = buf_load16(grs, row * C::ROWB + (2 * kc + h) * 16, 0);
  }
  const float my_lse2 = row < N ? lse2[int64_t(bh) * N + row] : 0.f;
  const float my_d = row < N ? Dv[int64_t(bh) * N + row] : 0.f;

  const TileLanes<C::CPR, C::ROWB> tl(lane);
  const int srow = tid / C::CPR, sch = tid % C::CPR;
  const int st_off0 = srow * C::ROWB + (sch ^ swz_both<C::CPR>(srow)) * 16;
  const int st_off1 =
      C::KFLIP ? srow * C::ROWB + (sch ^ swz_both<C::CPR>(srow + C::RSTEP)) * 16 : st_off0;
  auto st_off = [&](int i) { return (C::KFLIP && (i & 1)) ? st_off1 : st_off0; };
  constexpr int ST_STEP = C::NT * 16;
  const int dma_wave = wu * 1024;
  auto load_chunk = [&](int stage, int kt, int i) {
    buf_load16_lds(krs, Ks + stage * C::TILEB + dma_wave + i * ST_STEP, st_off(i),
                   kt * C::TILEB + i * ST_STEP);
    buf_load16_lds(vrs, Vs + stage * C::TILEB + dma_wave + i * ST_STEP, st_off(i),
                   kt * C::TILEB + i * ST_STEP);
  };
  auto load_tile = [&](int stage, int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) load_chunk(stage, kt, i);
  };
  // the next tile's loads ride one per k-step of the first block's S product
  static_assert(CPT <= C::KC, "one load per k-step");

  f32x16 dq[OB];
#pragma unroll
  for (int e = 0; e < OB; ++e) dq[e] = f32x16{};

  const int kt0 = rg * tps;                                       // first key tile
  const int nkt = min((N + C::BT - 1) / C::BT - kt0, tps);         // tiles of the range
  load_tile(0, kt0);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  lds_barrier();
  for (int kt = 0; kt < nkt; ++kt) {  // kt counts the range's tiles
    const int st = kt & 1;
    const bool more = kt + 1 < nkt;
    const int kb = st * C::TILEB;
#pragma unroll
    for (int t = 0; t < 2; ++t) {  // 32-key blocks of the tile
      // S^T = K Q^T and dP^T = V dO^T: keys 32t + (8(r/4) + 4h + r%4), query l32.  Keys
      // past N read zero K and V rows, so their dS meets a zero K row below and adds
      // nothing to dQ.
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int off = kb + tl.rb + 32 * t * C::ROWB + ((32 * kc) ^ tl.rx);
        s = mma16<BF16>(lds_read16(Ks, off), qf[kc], s);
        dp = mma16<BF16>(lds_read16(Vs, off), gf[kc], dp);
        if (t == 0 && more && kc < CPT) load_chunk(st ^ 1, kt0 + kt + 1, kc);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = ex2(fmaf(s[r], c, -my_lse2)) * (dp[r] - my_d);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int rb = 8 * x;
        const u32x4 sf = {pack16<BF16>(ds[rb + 0], ds[rb + 1]), pack16<BF16>(ds[rb + 2], ds[rb + 3]),
                          pack16<BF16>(ds[rb + 4], ds[rb + 5]), pack16<BF16>(ds[rb + 6], ds[rb + 7])};
        const int u = 2 * t + x;
#pragma unroll
        for (int e = 0; e < OB; ++e) {
          // dQ^T += K^T dS^T: K^T rows are the tile's key rows read transposed
          const int o0 = kb + tl.tb0 + 16 * u * C::ROWB + ((64 * e) ^ tl.tx);
          const int o1 = kb + tl.tb1 + 16 * u * C::ROWB + ((64 * e) ^ tl.tx);
          const u32x2 a0 = lds_read_tr(Ks, o0), a1 = lds_read_tr(Ks, o1);
          if constexpr (D == 256) {
            // dQ accumulates in AGPRs through assembly (fa_bwd_d256.hip keeps S and dP in
            // vector registers).  The first product of a key step reads dS packed just
            // before it: at least two wait states after that vector write.
            const u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
            if constexpr (BF16) {
              if (e == 0)
                asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                             : "+a"(dq[e]) : "v"(av), "v"(sf));
              else
                asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                             : "+a"(dq[e]) : "v"(av), "v"(sf));
            } else {
              if (e == 0)
                asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                             : "+a"(dq[e]) : "v"(av), "v"(sf));
              else
                asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                             : "+a"(dq[e]) : "v"(av), "v"(sf));
            }
          } else {
            dq[e] = mma16<BF16>(u32x4{a0[0], a0[1], a1[0], a1[1]}, sf, dq[e]);
          }
        }
      }
    }
    // the assembly products' latency is waited out inside the loop: the register
    // allocator may place copies of the accumulators at the loop's exit, ahead of any wait
    // written after it
    if constexpr (D == 256) mfma_drain();
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    lds_barrier();
  }

  if constexpr (D == 256) {
    // the assembly products' results: wait for the last, then fresh definitions
    mfma_drain();
#pragma unroll
    for (int e = 0; e < OB; ++e) asm volatile("" : "+a"(dq[e]));
    __builtin_amdgcn_sched_barrier(0);
  }
  constexpr int WAVE_LDS = (C::LDS / WAVES) & ~15;
  const int row0 = q0 + 32 * w;
  store_rows_lds<D, 1, false>(dq, 0.f, 1.f, 0.5f / scale, smem + w * WAVE_LDS,
                       dQ + slot + hoff + int64_t(row0) * D, nullptr, lane, N - row0);
}

// ------------------------------------------------------------------------------------

// nsplit ranges of tps streamed tiles each; dq, dk, dv receive nsplit slots of B H N d
// floats (with nsplit = 1 they are the gradients themselves).  The three steps are
// separate functions so that a head size's kernels can be instantiated in the unit whose
// code-generation choices suit them (fa_bwd_d128.hip, fa_bwd_d256.hip).
template <int D, bool BF16>
static hipError_t run_bwd_prep(const BwdProblem &p, hipStream_t stream) {
  const int64_t rows = int64_t(p.B) * p.H * p.N;
  const int64_t blocks = (rows * (D / 4) + 255) / 256;
  const int grid = int(blocks < kMaxGrid ? blocks : kMaxGrid);
  hipLaunchKernelGGL((fa_bwd_prep_kernel<D, BF16>), dim3(grid), dim3(256), 0, stream, p.o,
                     p.dout, p.lse, static_cast<uint16_t *>(p.ws_do16), p.ws_lse2, p.ws_d, rows);
  return hipGetLastError();
}

// dK and dV (WHAT = kDK | kDV), or one of them (d = 256: one launch for each)
template <int D, bool BF16, int WHAT>
static hipError_t run_bwd_dkdv(const BwdProblem &p, float *dk, float *dv, int nsplit, int tps,
                               hipStream_t stream) {
  constexpr int WAVES = 4;
  using C = CfgB<D, WAVES>;
  const int nb = (p.N + C::BR - 1) / C::BR;
  const int G = nb * p.B * p.H * nsplit;
  auto kern = fa_bwd_dkdv_kernel<D, BF16, WAVES, WHAT>;
  const hipError_t ea = allow_lds_on_device<fa_bwd_dkdv_kernel<D, BF16, WAVES, WHAT>>(C::LDS);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL(kern, dim3(G), dim3(C::NT), C::LDS, stream,
                     static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.k),
                     static_cast<const uint16_t *>(p.v),
                     static_cast<const uint16_t *>(p.ws_do16), p.ws_lse2, p.ws_d, dk, dv,
                     p.N, nb, G, p.scale * kLog2e, p.scale, nsplit, tps);
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t run_bwd_dq(const BwdProblem &p, float *dq, int nsplit, int tps,
                             hipStream_t stream) {
  constexpr int WAVES = 4;
  using C = CfgB<D, WAVES>;
  const int nb = (p.N + C::BR - 1) / C::BR;
  const int G = nb * p.B * p.H * nsplit;
  auto kern = fa_bwd_dq_kernel<D, BF16, WAVES>;
  const hipError_t ea = allow_lds_on_device<fa_bwd_dq_kernel<D, BF16, WAVES>>(C::LDS);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL(kern, dim3(G), dim3(C::NT), C::LDS, stream,
                     static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.k),
                     static_cast<const uint16_t *>(p.v),
                     static_cast<const uint16_t *>(p.ws_do16), p.ws_lse2, p.ws_d, dq, p.N,
                     nb, G, p.scale * kLog2e, p.scale, nsplit, tps);
  return hipGetLastError();
}

// the whole pass for d <= 128 (one key-owned launch for dK and dV)
template <int D, bool BF16>
static hipError_t run_bwd(const BwdProblem &p, float *dq, float *dk, float *dv, int nsplit,
                          int tps, hipStream_t stream) {
  static_assert(D <= 128, "d = 256 runs its dV, dK and dQ launches from two units");
  hipError_t e = run_bwd_prep<D, BF16>(p, stream);
  if (e == hipSuccess) e = run_bwd_dkdv<D, BF16, kDK | kDV>(p, dk, dv, nsplit, tps, stream);
  if (e == hipSuccess) e = run_bwd_dq<D, BF16>(p, dq, nsplit, tps, stream);
  return e;
}

}  // namespace fa
