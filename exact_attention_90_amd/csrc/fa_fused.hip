// Fused attention forward for gfx950 (FlashAttention forward pass).
//
// Algorithm: MUSA SDK guide "FlashAttention optimization", FlashAttention formula
// steps 1-4 / a-f, with the FlashAttention-2 split of the grid over Q blocks
// (same guide, "FlashAttention-2 improvement") and the Q-resident, K/V-streaming
// loop order of the pwwt.cn CK/MI50 notes (section 2.2).  Per workgroup:
//
//   prologue  Q tile [128 x d] -> LDS with coalesced 16-byte loads -> registers
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
// Layout of the work on the chip: 4 waves x 32 query rows.  Each wave computes S^T so
// that every lane owns ONE query row and 16 (of 32) keys per 32x32 block: the row
// max and row sum are in-lane reductions plus one exchange with lane ^ 32, and the
// rescale factor alpha is a per-lane scalar.  The P registers feed the P V product
// directly; V stays row-major in LDS and its operand is fetched with the
// transposing LDS load in the same key order the P registers hold.
#include <type_traits>

#include "fa_internal.h"
#include "fa_softmax.hpp"

namespace fa {

// ====================================================================================
// 16-bit inputs (binary16 or bfloat16), d in {64, 128, 256}
// ====================================================================================
template <int D, int WAVES>
struct Cfg16 {
  static constexpr int NT = 64 * WAVES;         // threads per workgroup
  static constexpr int BM = 32 * WAVES;         // query rows per workgroup (32 per wave)
  static constexpr int BN = 64;                 // keys per tile
  static constexpr int ROWB = D * 2;            // bytes per row
  static constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
  static constexpr int TILEB = BN * ROWB;       // bytes of one K or V tile
  static constexpr int CPT = TILEB / 16 / NT;   // chunks per thread per tile
  static constexpr int QCPT = BM * CPR / NT;    // Q chunks per thread
  static constexpr int SB = BN / 32;            // 32-key S blocks per tile
  static constexpr int KC = D / 16;             // k-steps of the Q K product
  static constexpr int OB = D / 32;             // 32-wide blocks of the output
  static constexpr int PU = BN / 16;            // k-steps of the P V product
  static constexpr int LDS = 4 * TILEB;         // K and V, two stages each
  // minimum waves per SIMD the registers must allow: at d = 256 one 32-row wave holds
  // O (128 registers) and Q (64) and needs more than half of the register file
  static constexpr int WPE = D == 256 ? 1 : 8 / WAVES;
  static_assert(CPT >= 1 && TILEB % (16 * NT) == 0, "a tile is whole chunks per thread");
  static_assert(BM * ROWB <= LDS, "Q staging must fit in the K and V stages");
  // the rows a thread moves differ by RSTEP per chunk.  The V swizzle key (period 4
  // rows) never changes; the K/Q key (period 16 rows) changes only when RSTEP is an odd
  // multiple of 8 (512-byte rows), and then alternates between two values
  static constexpr int RSTEP = NT / CPR;
  static constexpr bool KFLIP = RSTEP % 16 != 0;
  static_assert(RSTEP % 8 == 0, "thread row stride must keep the swizzle keys periodic");
};

template <int D, bool BF16, int WAVES>
__global__ __launch_bounds__(64 * WAVES, (Cfg16<D, WAVES>::WPE)) void fa_fwd16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, float *__restrict__ O, float *__restrict__ LSE, int N,
    int nqt, int G, float c, int nsplit, int kps) {
  using C = Cfg16<D, WAVES>;
  constexpr int SB = C::SB, OB = C::OB, PU = C::PU, CPT = C::CPT;
  constexpr int NA = SB * C::KC;  // matrix-core steps of S^T = K Q^T per tile
  constexpr int NB = OB * PU;     // matrix-core steps of O^T += V^T P^T per tile
  constexpr int DK = 4;           // K operand reads kept in flight
  constexpr int DV = 3;           // V operand reads (pairs) kept in flight
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char *const Ks = smem;
  char *const Vs = smem + 2 * C::TILEB;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  // workgroup L: Q tile L % nqt of key range (L / nqt) % nsplit of head L / (nqt nsplit).
  // Key range g holds keys [g kps, min(N, (g + 1) kps)); its result (O normalised over
  // those keys, and their LSE) goes to slot g of O and LSE, whose slots are B H N d and
  // B H N values apart.  With nsplit = 1 (kps = N) that is the whole attention.
  const int L = xcd_remap(blockIdx.x, G);
  const int qt = L % nqt, kg = (L / nqt) % nsplit, bh = L / nqt / nsplit;
  const int q0 = qt * C::BM;
  const int64_t hoff = int64_t(bh) * N * D;
  const int64_t bhn = int64_t(G / (nqt * nsplit)) * N;  // rows of one output slot
  const int kbeg = kg * kps, NK = min(N - kbeg, kps);    // keys of this range, >= 1
  // buffer resources over this head's [N, D] slices (K and V: the range's rows): loads
  // past the last row read zeros
  const uint32_t head_bytes = uint32_t(N) * C::ROWB;
  const auto qrs = make_rsrc(Q + hoff, head_bytes);
  const auto krs = make_rsrc(K + hoff + int64_t(kbeg) * D, uint32_t(NK) * C::ROWB);
  const auto vrs = make_rsrc(V + hoff + int64_t(kbeg) * D, uint32_t(NK) * C::ROWB);
  constexpr int ST_STEP = C::NT * 16;  // bytes between a thread's chunks, in LDS and memory
  // A tile of rows is one contiguous block of global memory: thread tid moves the
  // 16-byte chunks tid + NT i.  Their LDS rows differ by NT/CPR per i, which leaves
  // the swizzle key unchanged, so one lane offset plus immediates addresses them all.
  // With 512-byte rows the swizzle key of odd chunks is the other of two values.
  const int srow = tid / C::CPR, sch = tid % C::CPR;
  const int st_k = srow * C::ROWB + swz_row<C::CPR>(srow, sch) * 16;
  const int st_k1 =
      C::KFLIP ? srow * C::ROWB + swz_row<C::CPR>(srow + C::RSTEP, sch) * 16 : st_k;
  auto st_ki = [&](int i) { return (C::KFLIP && (i & 1)) ? st_k1 : st_k; };

  // ---- prologue: Q tile -> LDS (coalesced 16-byte loads) -> registers ----
#pragma unroll
  for (int i = 0; i < C::QCPT; ++i)
    lds_write16(Ks, st_ki(i) + i * ST_STEP, buf_load16(qrs, tid * 16, q0 * C::ROWB + i * ST_STEP));
  __syncthreads();
  u32x4 qf[C::KC];
  {
    const int qr = 32 * w + l32;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc)
      qf[kc] = lds_read16(Ks, qr * C::ROWB + swz_row<C::CPR>(qr, 2 * kc + h) * 16);
  }
  __syncthreads();

  // ---- per-lane LDS offsets, fixed for the whole loop ----
  const int st_v = srow * C::ROWB + swz_v<C::CPR>(srow, sch) * 16;
  // K operand rows 32t + l32 at logical chunk 2 kc + h: the XOR swizzle key k of row l32
  // splits as chunk (2 kc + h) ^ k = 2 (kc ^ (k >> 1)) + (h ^ (k & 1)), so the byte offset
  // is k_base + ((32 kc) ^ k_xor), one xor-add per k-step instead of KC live registers
  int k_base, k_xor;
  {
    const int key = swz_row<C::CPR>(l32, 0);  // the key itself (chunk 0 ^ key)
    k_base = l32 * C::ROWB + (h ^ (key & 1)) * 16;
    k_xor = (key >> 1) * 32;
  }
  // transposing V reads: lane j of 16-lane group G reads key row 16u + 8x + 4(G/2) + j/4
  // at columns 32e + 16(G%2) + 4(j%4).  Column chunk 4e + c0 (c0 < 4) of row r sits at
  // chunk (4e + c0) ^ 4 k(r) = 4 (e ^ k) + c0, so the byte offset is
  // v_base + ((64 e) ^ v_xor) with lane constants v_base and v_xor
  int v_base, v_xor;
  {
    const int grp = lane >> 4, j16 = lane & 15;
    const int vrow0 = 4 * (grp >> 1) + (j16 >> 2);
    const int vcol0 = 16 * (grp & 1) + 4 * (j16 & 3);
    const int c0 = vcol0 >> 3;
    v_base = vrow0 * C::ROWB + c0 * 16 + (vcol0 & 7) * 2;
    v_xor = (swz_v<C::CPR>(vrow0, c0) ^ c0) * 16;  // 64 k(r): the swizzle's xor term
  }

  // ---- K/V tile movement ----
  // K and V tiles go from global memory straight into an LDS stage.  LDS byte 16 c of a
  // stage is written by lane c % 64 of wave (c / 64) % WAVES, instruction c / NT; that
  // position holds logical chunk swz(row, c % CPR) of row c / CPR, and since each swizzle
  // is an involution the lane's global offset within the tile is its st_k / st_v value.
  // Tiles past the end of the head read as zeros (buffer range check), so loads are
  // issued unconditionally; their offsets stay below 2^31 for every accepted shape.
  const int dma_wave = __builtin_amdgcn_readfirstlane(w) * 1024;  // wave's 1 KiB of a step
  auto dma_k = [&](char *kb, int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      buf_load16_lds(krs, kb + dma_wave + i * ST_STEP, st_ki(i), kt * C::TILEB + i * ST_STEP);
  };
  auto dma_v = [&](char *vb, int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      buf_load16_lds(vrs, vb + dma_wave + i * ST_STEP, st_v, kt * C::TILEB + i * ST_STEP);
  };
  // bfloat16 V: the P V product runs in binary16, so each thread widens the chunks its
  // own loads wrote (chunk i: 16 bytes at dma_wave + i ST_STEP + 16 lane), in place.
  // Needs only this wave's loads to have landed; other waves read the stage after the
  // barrier that ends the iteration.
  auto widen_v = [&](char *vb, int i) {
    if constexpr (BF16) {
      char *p = vb + dma_wave + i * ST_STEP;
      u32x4 vv = lds_read16(p, lane * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) vv[q] = bf16x2_to_f16x2(vv[q]);
      lds_write16(p, lane * 16, vv);
    }
  };
  // operand of matrix-core step i: S^T step i = (block t = i / KC, k-step i % KC);
  // P V step i = (output block e = i % OB, key step u = i / OB).  kb / vb are the lane's
  // base offsets into the K / V stage being read (stage offset + k_base / v_base).
  auto k_op = [&](int kb, int i) {
    const int t = i / C::KC, kc = i % C::KC;  // block-major: all k-steps of block 0 first
    const int off = kb + ((32 * kc) ^ k_xor) + 32 * t * C::ROWB;
    return lds_read16(smem, off);
  };
  auto v_op = [&](int vb, int i) {
    const int u = i / OB, e = i % OB;
    const int off = vb + ((64 * e) ^ v_xor);
    const u32x2 a0 = lds_read_tr(smem, off + (16 * u) * C::ROWB);
    const u32x2 a1 = lds_read_tr(smem, off + (16 * u + 8) * C::ROWB);
    return u32x4{a0[0], a0[1], a1[0], a1[1]};
  };

  f32x16 o[OB];
#pragma unroll
  for (int e = 0; e < OB; ++e) o[e] = f32x16{};
  // online-softmax state of the lane's query row: running max (base-2 units), this
  // lane's partial row sum, and, for the tile whose P is pending, its rescale factor
  // alpha and P row sum; lazy form only: the partial sums of P as rounded to binary16
  // for the P V product (lp, and rp for the pending tile)
  float mc = -INFINITY, l = 0.f, alpha = 0.f, rs = 0.f, lp = 0.f, rp = 0.f;
  const int nkt = (NK + C::BN - 1) / C::BN;
  const int nlast = NK - (nkt - 1) * C::BN;  // valid keys of the last tile, 1 .. BN

  // ---- the softmax of one tile is split across the two halves of an iteration ----
  // S^T holds 32 scores per lane: block 0 (keys 0-31 of the tile, registers s[0]) and
  // block 1 (keys 32-63, s[1]); score x is s[x / 16][x % 16].
  //   during B (the P V product of the previous tile): the row max over all 32 scores,
  //     the new running max and alpha, then P = 2^(c s - c m) for block 0, which is packed
  //     into operand blocks 0 and 1 as soon as the previous tile's P V steps release them
  //   during A (the S product of the next tile, which rebuilds s[0] first and s[1] last):
  //     P for block 1, packed into operand blocks 2 and 3 before s[1] is overwritten, the
  //     row sum, l = alpha l + sum, and O = alpha O
  // The row sum adds the 32 values of P in score order, as a single pass would.
  //
  // At d = 256 the output accumulators live in the matrix-core (AGPR) registers, where a
  // multiply costs a read, the multiply and a write per element.  There the reference
  // max mc moves only when a tile's row max exceeds it by more than kTau (base-2 units):
  // P <= 2^kTau stays far inside binary16 range, softmax is unchanged by the choice of
  // reference, and most tiles leave every alpha at 1, so O is rescaled in a wave-uniform
  // branch that is rarely taken.  P > 1 then carries the binary16 rounding of values
  // that are not powers of two even for the row's largest score, so O is normalised by
  // the sum of P as rounded for the P V product (the weights applied to V sum to one)
  // and LSE by the exact sum.
  constexpr bool LAZY = D == 256;
  constexpr float kTau = 8.0f;
  constexpr int KC = C::KC;
  constexpr int NMX = NB >= 16 ? 2 : 1;  // B steps of the row max
  constexpr int NEB = NB - NMX - 1;      // B steps carrying block-0 exponentials
  constexpr int NEA = KC - 1;            // A steps carrying block-1 exponentials
  float mx = 0.f, sub = 0.f;
  auto max_step = [&](f32x16 (&s)[SB], int k) {
    const int b = k * 32 / NMX, e = (k + 1) * 32 / NMX;
    if (k == 0) mx = s[0][0];
#pragma unroll
    for (int x = 0; x < 32; ++x)
      if (x >= b && x < e) mx = fmaxf(mx, s[x / 16][x % 16]);
  };
  auto finalize_max = [&]() {
    mx = pair_max(mx);  // full row max over the tile's keys
    // running max in base-2 units (lazy: the reference, moved only past mc + kTau;
    // -inf + kTau stays -inf, so the first tile with a valid key always sets it)
    const float mxc = mx * c;
    const float mc_new = LAZY ? (mxc > mc + kTau ? mxc : mc) : fmaxf(mc, mxc);
    // a row that has seen only masked keys keeps alpha = 0 and P = 0 (no inf - inf)
    alpha = (mc == -INFINITY) ? 0.f : ex2(mc - mc_new);
    sub = (mc_new == -INFINITY) ? 0.f : mc_new;
    mc = mc_new;
    rs = 0.f;
    rp = 0.f;
  };
  auto exp_range = [&](f32x16 (&s)[SB], int b, int e) {
#pragma unroll
    for (int x = 0; x < 32; ++x)
      if (x >= b && x < e) {
        const float p = ex2(fmaf(s[x / 16][x % 16], c, -sub));
        s[x / 16][x % 16] = p;
        rs += p;
      }
  };
  // keys at or past nvalid of a tile are masked to -inf before its softmax
  auto mask = [&](f32x16 (&s)[SB], int nvalid) {
#pragma unroll
    for (int t = 0; t < SB; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
        if (key >= nvalid) s[t][r] = -INFINITY;
      }
  };
  // P (fp32, S^T register layout) -> binary16 operands: step u takes block u/2,
  // registers 8(u%2) .. +7, i.e. keys 16u + 8x + 4h + s for slot 4x + s
  u32x4 pf[PU];
  auto pack_u = [&](const f32x16 (&s)[SB], int u) {
    const int t = u >> 1, rb = (u & 1) * 8;
    pf[u] = u32x4{pack_f16(s[t][rb + 0], s[t][rb + 1]), pack_f16(s[t][rb + 2], s[t][rb + 3]),
                  pack_f16(s[t][rb + 4], s[t][rb + 5]), pack_f16(s[t][rb + 6], s[t][rb + 7])};
    pin(pf[u]);
    if constexpr (LAZY) rp = sum8_f16(pf[u], rp);
  };
  // B step k's share of the softmax; operand block u (0 or 1) is packed at the first
  // step where its 8 exponentials are done and its last reader (step OB u + OB - 1) of the
  // previous tile's P V product has issued
  auto b_exp_end = [](int k) { return k <= NMX ? 0 : (k - NMX) * 16 / NEB; };
  auto b_pack_step = [&](int u) {
    int k = NMX + 1;
    while (b_exp_end(k) < 8 * u + 8) ++k;
    return k > OB * u + OB ? k : OB * u + OB;
  };
  auto soft_b = [&](f32x16 (&s)[SB], int k) {
    if (k < NMX) max_step(s, k);
    else if (k == NMX) finalize_max();
    else exp_range(s, b_exp_end(k - 1), b_exp_end(k));
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (b_pack_step(u) == k) pack_u(s, u);
  };
  // A step k's share: block-1 exponentials on steps 0 .. NEA-1, then (step NEA) the last
  // two operand blocks and l; O = alpha O on the steps that rebuild s[1]
  auto soft_a = [&](f32x16 (&s)[SB], int k) {
    if (k < NEA) exp_range(s, 16 + k * 16 / NEA, 16 + (k + 1) * 16 / NEA);
    if (k == NEA) {
      pack_u(s, 2);
      pack_u(s, 3);
      l = fmaf(l, alpha, rs);
      if constexpr (LAZY) lp = fmaf(lp, alpha, rp);
    }
    if (!LAZY && k >= KC) {
      constexpr int R = OB * 16 / KC;
      const int q = k - KC;
#pragma unroll
      for (int x = 0; x < OB * 16; ++x)
        if (x >= q * R && x < (q + 1) * R) o[x / 16][x % 16] *= alpha;
      pin(o[q * R / 16]);
    }
  };

  // lazy form: O = alpha O for the whole tile, skipped when every alpha of the wave is 1
  auto rescale_lazy = [&]() __attribute__((always_inline)) {
    if constexpr (LAZY) {
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int e = 0; e < OB; ++e)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[e][r] *= alpha;
      }
    }
  };

  // S of the tile being started (becomes its P in place); the packed P of the tile
  // whose P V product is pending lives in pf
  f32x16 s[SB];
  u32x4 kf[DK], vf[DV];
  // S product step i, block-major so s[0] is rebuilt before s[1]
  auto s_step = [&](int kb, int i, u32x4 kop) {
    const int t = i / KC, kc = i % KC;
    s[t] = mma16<BF16>(kop, qf[kc], kc == 0 ? f32x16{} : s[t]);
  };

  // Loads into LDS are waited for explicitly: each wave waits (s_waitcnt vmcnt, loads
  // retire in issue order) for its own loads of the stages the next barrier publishes,
  // and leaves the younger ones in flight.
  auto wait_loads = [](auto n) {  // at most n.value of this wave's loads in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_only(decltype(n)::value));
  };
  using in_flight_0 = std::integral_constant<int, 0>;
  using in_flight_1 = std::integral_constant<int, CPT>;  // one tile of K or V

  // ---- prologue: K_0, V_0 and K_1 staged; S_0 and the B share of its softmax ----
  dma_k(Ks, 0);
  dma_v(Vs, 0);
  dma_k(Ks + C::TILEB, 1);
  wait_loads(in_flight_1{});  // K_0 and V_0 have landed
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) widen_v(Vs, i);
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < NA; ++i) s_step(k_base, i, k_op(k_base, i));
  if (nkt == 1 && nlast < C::BN) mask(s, nlast);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    soft_b(s, k);
    __builtin_amdgcn_sched_barrier(0);
  }
  // K_1 has landed, and every wave is done with K_0 before stage 0 is refilled
  wait_loads(in_flight_0{});
  lds_barrier();

  // ---- steady state: iteration j (P = j % 2 selects the LDS stages) ----
  //   A: V_{j+1} and K_{j+2} start towards LDS; S_{j+1} = K_{j+1} Q^T on the matrix
  //      cores, while the VALU finishes the softmax of tile j and rescales O by alpha_j
  //   B: O += V_j P_j on the matrix cores, while the VALU starts the softmax of S_{j+1}
  //      and widens bfloat16 V_{j+1}
  // The stages written in iteration j held K_j and V_{j-1}, last read in iteration j-1;
  // the barrier that ends each iteration orders every stage's last read before its next
  // write, and every write before its next read: before it each wave waits for its loads
  // of V_{j+1} and K_{j+2}, which iteration j + 1 reads.  B waits for V_{j+1} alone (it
  // was issued first) before widening it, and the transposing reads of V_j wait for
  // nothing.
  // MASKED: the tile started in this iteration (j + 1) is the last one, so its keys past
  // N are masked; only the final iteration is compiled with it, keeping the mask out of
  // the steady-state loop
  auto iter = [&](int j, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const int P = j & 1;
    // lane bases of this iteration's reads (the pins keep the offset arithmetic inside
    // the loop rather than precomputed into live registers)
    pin(k_xor);
    pin(v_xor);
    const int kb = k_base + (1 - P) * C::TILEB;         // K_{j+1}
    const int vb = v_base + (2 + P) * C::TILEB;         // V_j
    char *vw = Vs + (1 - P) * C::TILEB;                 // V_{j+1}, widened in B
    char *kw = Ks + P * C::TILEB;                       // K_{j+2}

    // ---- A ----
    dma_v(vw, j + 1);
    dma_k(kw, j + 2);
    rescale_lazy();
#pragma unroll
    for (int i = 0; i < DK; ++i) kf[i] = k_op(kb, i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      s_step(kb, i, kf[i % DK]);
      if (i + DK < NA) kf[i % DK] = k_op(kb, i + DK);
      soft_a(s, i);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- B ----
#pragma unroll
    for (int i = 0; i < DV; ++i) vf[i] = v_op(vb, i);
    if (MASKED && nlast < C::BN) mask(s, nlast);
    // bfloat16 V_{j+1} is widened in place during the P V product below, once this
    // wave's loads of it have landed (the loads issued after it may stay in flight)
    if constexpr (BF16) wait_loads(in_flight_1{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int u = i / OB, e = i % OB;
      o[e] = mma_f16(vf[i % DV], pf[u], o[e]);
      if (i + DV < NB) vf[i % DV] = v_op(vb, i + DV);
      soft_b(s, i);
      if (i % (NB / CPT) == NB / CPT - 1) widen_v(vw, i / (NB / CPT));
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_loads(in_flight_0{});
    lds_barrier();
  };

  for (int j = 0; j + 2 < nkt; ++j) iter(j, std::false_type{});
  if (nkt >= 2) iter(nkt - 2, std::true_type{});

  // ---- last tile T = nkt - 1: the A share of its softmax, then its P V product ----
  {
    const int vb = v_base + (2 + ((nkt - 1) & 1)) * C::TILEB;
    rescale_lazy();
#pragma unroll
    for (int k = 0; k < NA; ++k) soft_a(s, k);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int u = i / OB, e = i % OB;
      o[e] = mma_f16(v_op(vb, i), pf[u], o[e]);
    }
  }

  // every wave is done with the K/V stages before they hold the output
  lds_barrier();
  constexpr int WAVE_LDS = C::LDS / WAVES;                 // bytes of a wave's region
  constexpr int NHALF = (32 * D * 4 + WAVE_LDS - 1) / WAVE_LDS;
  const int row0 = q0 + 32 * w;  // the wave's first query row
  store_rows_lds<D, NHALF>(o, mc, l, LAZY ? lp : l, smem + w * WAVE_LDS,
                           O + kg * bhn * D + hoff + int64_t(row0) * D,
                           LSE + kg * bhn + int64_t(bh) * N + row0, lane, N - row0);
}

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

template <int D>
__global__ __launch_bounds__(256, 1) void fa_fwd32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, int N, int nqt, int G, float c, int nsplit,
    int kps) {
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

// Waves per workgroup of the 16-bit kernel: at d = 128, eight waves (256 query rows)
// halve the K/V tile loads and the bfloat16 widening per query row; at d = 64 the
// softmax dominates and four waves schedule better; at d = 256 a wave needs more than
// half a SIMD's registers, so four waves (one per SIMD) are all a compute unit holds.
template <int D>
constexpr int waves16() { return D == 128 ? 8 : 4; }

// nsplit key ranges of kps keys each (the last may be shorter, none is empty); with
// nsplit = 1 and kps = N the kernel writes the attention itself to o and lse
template <int D, bool BF16, int WAVES = waves16<D>()>
static hipError_t run16(const Problem &p, float *o, float *lse, int nsplit, int kps,
                        hipStream_t stream) {
  using C = Cfg16<D, WAVES>;
  auto kern = fa_fwd16_kernel<D, BF16, WAVES>;
  const hipError_t ea = allow_lds_on_device<fa_fwd16_kernel<D, BF16, WAVES>>(C::LDS);
  if (ea != hipSuccess) return ea;
  const int nqt = (p.N + C::BM - 1) / C::BM;
  const int G = nqt * p.B * p.H * nsplit;
  const float c = p.scale * kLog2e;
  hipLaunchKernelGGL(kern, dim3(G), dim3(C::NT), C::LDS, stream,
                     static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.k),
                     static_cast<const uint16_t *>(p.v), o, lse, p.N, nqt, G, c, nsplit, kps);
  return hipGetLastError();
}

template <bool BF16>
static hipError_t run16_any(const Problem &p, float *o, float *lse, int nsplit, int kps,
                            hipStream_t stream) {
  return p.d == 256 ? run16<256, BF16>(p, o, lse, nsplit, kps, stream)
         : p.d == 128 ? run16<128, BF16>(p, o, lse, nsplit, kps, stream)
                      : run16<64, BF16>(p, o, lse, nsplit, kps, stream);
}

template <int D>
static hipError_t run32(const Problem &p, float *o, float *lse, int nsplit, int kps,
                        hipStream_t stream) {
  using C = Cfg32<D>;
  auto kern = fa_fwd32_kernel<D>;
  const hipError_t ea = allow_lds_on_device<fa_fwd32_kernel<D>>(C::LDS);
  if (ea != hipSuccess) return ea;
  const int nqt = (p.N + C::BM - 1) / C::BM;
  const int G = nqt * p.B * p.H * nsplit;
  const float c = p.scale * kLog2e;
  hipLaunchKernelGGL(kern, dim3(G), dim3(256), C::LDS, stream,
                     static_cast<const float *>(p.q), static_cast<const float *>(p.k),
                     static_cast<const float *>(p.v), o, lse, p.N, nqt, G, c, nsplit, kps);
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
      return run16_any<false>(p, p.o, p.lse, 1, p.N, stream);
    case kBF16:
      return run16_any<true>(p, p.o, p.lse, 1, p.N, stream);
    default:
      return run32_any(p, p.o, p.lse, 1, p.N, stream);
  }
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
  hipError_t e = p.dtype == kBF16  ? run16_any<true>(p, opart, lpart, nsplit, kps, stream)
                 : p.dtype == kF16 ? run16_any<false>(p, opart, lpart, nsplit, kps, stream)
                                   : run32_any(p, opart, lpart, nsplit, kps, stream);
  if (e != hipSuccess) return e;
  return p.d == 256 ? run_merge<256>(p, opart, lpart, nsplit, stream)
         : p.d == 128 ? run_merge<128>(p, opart, lpart, nsplit, stream)
                      : run_merge<64>(p, opart, lpart, nsplit, stream);
}

}  // namespace fa
