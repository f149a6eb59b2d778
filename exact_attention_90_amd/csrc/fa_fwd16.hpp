// 16-bit (binary16 / bfloat16) fused attention forward kernel for gfx950, as a template:
// its instantiations are compiled in fa_fwd16.hip (d = 64, 256) and fa_fwd16_d128.hip
// (d = 128, whose code generation takes different compiler options).
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
// Layout of the work on the chip: WAVES waves x RB blocks of 32 query rows (8 x 1 at
// d = 128, 4 x 2 at d = 64, 4 x 1 at d = 256).  Each wave computes S^T so that every
// lane owns ONE query row of a block and 16 (of 32) keys per 32x32 block: the row
// max and row sum are in-lane reductions plus one exchange with lane ^ 32, and the
// rescale factor alpha is a per-lane scalar.  The P registers feed the P V product
// directly; V stays row-major in LDS and its operand is fetched with the
// transposing LDS load in the same key order the P registers hold.
#pragma once

#include <type_traits>

#include "fa_internal.h"
#include "fa_softmax.hpp"

namespace fa {

// ====================================================================================
// 16-bit inputs (binary16 or bfloat16), d in {64, 128, 256}
// ====================================================================================
template <int D, int WAVES, int RB>
struct Cfg16 {
  static constexpr int NT = 64 * WAVES;         // threads per workgroup
  static constexpr int BM = 32 * RB * WAVES;    // query rows per workgroup (32 RB per wave)
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
  static constexpr int QB = BM * ROWB;          // bytes of a Q tile
  // persistent form: plus a Q region (d = 256: half of one, beside 128 KiB of K/V stages
  // in the 160 KiB of LDS; the other half of the next Q goes to a K stage)
  static constexpr int LDSP = LDS + (D == 256 ? QB / 2 : QB);
  // minimum waves per SIMD the registers must allow: at d = 256 one 32-row wave holds
  // O (128 registers) and Q (64), and a wave of two 32-row blocks at d = 128 holds two
  // of each; both need more than half of the register file.  Two 32-row blocks at d = 64
  // (O 64, Q 32, S 64, P 32) fit two waves per SIMD.
  static constexpr int WPE = (D == 256 || (RB == 2 && D > 64)) ? 1 : RB == 2 ? 2 : 8 / WAVES;
  static_assert(CPT >= 1 && TILEB % (16 * NT) == 0, "a tile is whole chunks per thread");
  static_assert(BM * ROWB <= LDS, "Q staging must fit in the K and V stages");
  // the rows a thread moves differ by RSTEP per chunk.  The V swizzle key (period 4
  // rows) never changes; the K/Q key (period 16 rows) changes only when RSTEP is an odd
  // multiple of 8 (512-byte rows), and then alternates between two values
  static constexpr int RSTEP = NT / CPR;
  static constexpr bool KFLIP = RSTEP % 16 != 0;
  static_assert(RSTEP % 8 == 0, "thread row stride must keep the swizzle keys periodic");
};

// With two query blocks per wave, or at d = 256, the P V products are written as
// assembly that accumulates in the matrix-core (AGPR) registers (mfma_drain, in
// fa_device.hpp, covers the latency the compiler does not track), and the packed P
// operands are written at least one whole matrix-core step before a product reads them
// (scheduling fences separate the pipeline steps; after the last tile's softmax a drain
// separates them).

// RB = 32-row query blocks per wave.  With RB = 2 every K operand read from LDS feeds
// the S products of both blocks and every V operand read feeds both P V products, which
// halves the LDS operand bytes per flop.  At d = 64 the two blocks fit two waves per SIMD
// in vector registers; at d = 128 their output accumulators need the matrix-core (AGPR)
// registers, and one wave runs per SIMD.
//
// STATS: the statistics-recording form (validation only, nsplit = 1): after every key
// tile t each query row's running max (base-2 units, c m) and row sum go to
// ST[((b H + h) N + i) ceil(N/64) + t][0..1].  The other forms ignore ST.
//
// PERSIST: the persistent form (d = 128 or 256, one block per wave, nsplit = 1, at least
// two key tiles, no STATS).  The grid holds fewer workgroups than the G tiles and
// workgroup b takes tiles b, b + gridDim.x, b + 2 gridDim.x, ... in turn.  The next tile's
// Q (d = 128: into an LDS region of its own; d = 256: half there, half into a freed K
// stage) and its first K and V tiles are loaded while the current tile's last key tiles
// are processed, so that a new tile starts without waiting for memory, and its output
// goes out through LDS that the next tile's first K/V tiles do not occupy.
template <int D, bool BF16, int WAVES, int RB, bool STATS = false, bool PERSIST = false>
__global__ __launch_bounds__(64 * WAVES, (Cfg16<D, WAVES, RB>::WPE)) void fa_fwd16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, float *__restrict__ O, float *__restrict__ LSE, int N,
    int nqt, int G, float c, int nsplit, int kps, float *__restrict__ ST) {
  using C = Cfg16<D, WAVES, RB>;
  constexpr int SB = C::SB, OB = C::OB, PU = C::PU, CPT = C::CPT;
  constexpr int NA = SB * C::KC;  // matrix-core steps of S^T = K Q^T per tile
  constexpr int NB = OB * PU;     // matrix-core steps of O^T += V^T P^T per tile
  // every chunk of the next tiles' loads gets an S step of its own, and each chunk's
  // widening a read step before its write step
  static_assert(NA >= 2 * CPT, "the A half issues 2 CPT load chunks, one per step");
  static_assert(NB % CPT == 0 && NB / CPT >= 2, "widening: read and write steps per chunk");
  // K operand reads and V operand read pairs kept in flight (fewer for two blocks at
  // d = 64, which must fit two waves per SIMD)
  constexpr int DK = (D == 64 && RB == 2) ? 3 : 4;
  constexpr int DV = (D == 64 && RB == 2) ? 2 : 3;
  constexpr bool PAIRW = RB == 1;
  auto imin = [](int a, int b) __attribute__((always_inline)) { return a < b ? a : b; };
  // LDS accesses of the bfloat16 widening issued in P V steps a .. b-1 (chunk reads on
  // steps 1 mod NB/CPT, writes on steps -1 mod NB/CPT)
  auto widen_ops = [](int a, int b) __attribute__((always_inline)) {
    int n = 0;
    if constexpr (BF16)
      for (int k = a < 0 ? 0 : a; k < b; ++k)
        n += (k % (NB / CPT) == 1) + (k % (NB / CPT) == NB / CPT - 1);
    return n;
  };
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char *const Ks = smem;
  char *const Vs = smem + 2 * C::TILEB;
  // the Q tile is staged in the K stages, or in the persistent form at d = 128 in a region
  // of its own.  QSPLIT (the persistent form at d = 256): the next tile's Q rows 0 .. BM/2-1
  // go to the region past the K/V stages (Xs, half a Q tile), rows BM/2 .. BM-1 to the K
  // stage its last key tile has left.
  constexpr bool QSPLIT = PERSIST && D == 256;
  char *const Qs = (PERSIST && !QSPLIT) ? smem + C::LDS : smem;
  constexpr int XS_OFF = C::LDS;  // byte offset of Xs in LDS
  static_assert(!PERSIST || !STATS, "the persistent form records no statistics");

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  // workgroup L: Q tile L % nqt of key range (L / nqt) % nsplit of head L / (nqt nsplit).
  // Key range g holds keys [g kps, min(N, (g + 1) kps)); its result (O normalised over
  // those keys, and their LSE) goes to slot g of O and LSE, whose slots are B H N d and
  // B H N values apart.  With nsplit = 1 (kps = N) that is the whole attention.
  const int64_t bhn = int64_t(G / (nqt * nsplit)) * N;  // rows of one output slot
  const uint32_t head_bytes = uint32_t(N) * C::ROWB;
  int vt = blockIdx.x;  // the workgroup's tile (in the persistent form, the current one)
  int qt, kg, bh, q0, kbeg;
  int64_t hoff;
  // buffer resources over this head's [N, D] slices (K and V: the range's rows): loads
  // past the last row read zeros
  __amdgpu_buffer_rsrc_t qrs, krs, vrs;
  auto set_tile = [&](int v) __attribute__((always_inline)) {
    const int L = xcd_remap(v, G);
    qt = L % nqt;
    kg = (L / nqt) % nsplit;
    bh = L / nqt / nsplit;
    q0 = qt * C::BM;
    hoff = int64_t(bh) * N * D;
    kbeg = kg * kps;
    const int nk = min(N - kbeg, kps);  // keys of this range, >= 1
    qrs = make_rsrc(Q + hoff, head_bytes);
    krs = make_rsrc(K + hoff + int64_t(kbeg) * D, uint32_t(nk) * C::ROWB);
    vrs = make_rsrc(V + hoff + int64_t(kbeg) * D, uint32_t(nk) * C::ROWB);
  };
  set_tile(vt);
  // keys of the range (in the persistent form, nsplit = 1: N for every tile)
  const int NK = min(N - kbeg, kps);
  // persistent form: the next tile.  For the workgroup's last tile the same loads are
  // issued (so that every wait counts the same loads) over an empty buffer range: they
  // read nothing from memory and write zeros to LDS regions that nothing reads any more.
  bool has_next = false;
  int q0n = 0;
  __amdgpu_buffer_rsrc_t qrn = qrs, krn = krs, vrn = vrs;
  auto set_next = [&]() __attribute__((always_inline)) {
    has_next = vt + int(gridDim.x) < G;
    const int L = xcd_remap(has_next ? vt + int(gridDim.x) : vt, G);
    const int64_t ho = int64_t(L / nqt) * N * D;
    const uint32_t nb = has_next ? head_bytes : 0u;
    q0n = (L % nqt) * C::BM;
    qrn = make_rsrc(Q + ho, nb);
    krn = make_rsrc(K + ho, nb);
    vrn = make_rsrc(V + ho, nb);
  };
  constexpr int ST_STEP = C::NT * 16;  // bytes between a thread's chunks, in LDS and memory
  // A tile of rows is one contiguous block of global memory: thread tid moves the
  // 16-byte chunks tid + NT i.  Their LDS rows differ by NT/CPR per i, which leaves
  // the swizzle key unchanged, so one lane offset plus immediates addresses them all.
  // With 512-byte rows the swizzle key of odd chunks is the other of two values.
  const int srow = tid / C::CPR, sch = tid % C::CPR;
  const int st_k = srow * C::ROWB + swz_row<C::CPR>(srow, sch) * 16;
  const int st_k1 =
      C::KFLIP ? srow * C::ROWB + swz_row<C::CPR>(srow + C::RSTEP, sch) * 16 : st_k;
  auto st_ki = [&](int i) __attribute__((always_inline)) { return (C::KFLIP && (i & 1)) ? st_k1 : st_k; };

  // ---- prologue: Q tile -> LDS (coalesced 16-byte loads) -> registers ----
#pragma unroll
  for (int i = 0; i < C::QCPT; ++i)
    lds_write16(Qs, st_ki(i) + i * ST_STEP, buf_load16(qrs, tid * 16, q0 * C::ROWB + i * ST_STEP));
  __syncthreads();
  // block r of wave w holds query rows 32 (RB w + r) .. +31 of the tile
  u32x4 qf[RB][C::KC];
  // base: LDS byte offset of the tile's row 0 (row qr at base + qr ROWB, swizzled chunks)
  auto read_q = [&](int base) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int qr = 32 * (RB * w + r) + l32;
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc)
        qf[r][kc] =
            lds_read16(smem, base + qr * C::ROWB + swz_row<C::CPR>(qr, 2 * kc + h) * 16);
    }
  };
  read_q(int(Qs - smem));
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
  auto dma_k = [&](char *kb, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      buf_load16_lds_off<PERSIST>(krs, kb + dma_wave + i * ST_STEP, st_ki(i), kt * C::TILEB,
                                  i * ST_STEP);
  };
  auto dma_v = [&](char *vb, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      buf_load16_lds_off<PERSIST>(vrs, vb + dma_wave + i * ST_STEP, st_v, kt * C::TILEB,
                                  i * ST_STEP);
  };
  // one chunk of a tile's load: an iteration's loads ride one per step between its
  // first matrix-core steps instead of all issuing before them (measured: bitwise the
  // same results, +2.7 % at bf16 8x32x4096x128, +3.9 % at d = 256)
  // (safe: the form that keeps the scalar operands' wait states, for the steps where the
  // persistent form restores spilled scalars; the steady-state loop has none)
  auto dma_k1 = [&](char *kb, int kt, int i, auto safe) __attribute__((always_inline)) {
    buf_load16_lds_off<decltype(safe)::value>(krs, kb + dma_wave + i * ST_STEP, st_ki(i),
                                              kt * C::TILEB, i * ST_STEP);
  };
  auto dma_v1 = [&](char *vb, int kt, int i, auto safe) __attribute__((always_inline)) {
    buf_load16_lds_off<decltype(safe)::value>(vrs, vb + dma_wave + i * ST_STEP, st_v,
                                              kt * C::TILEB, i * ST_STEP);
  };
  // the persistent form's loads of the next tile: chunk i of its K or V tile kt, and
  // chunk i of its Q tile into the Q region (the same swizzled layout as the Q prologue)
  auto dma_kn = [&](char *kb, int kt, int i) __attribute__((always_inline)) {
    buf_load16_lds_off<PERSIST>(krn, kb + dma_wave + i * ST_STEP, st_ki(i), kt * C::TILEB,
                                i * ST_STEP);
  };
  auto dma_vn = [&](char *vb, int kt, int i) __attribute__((always_inline)) {
    buf_load16_lds_off<PERSIST>(vrn, vb + dma_wave + i * ST_STEP, st_v, kt * C::TILEB,
                                i * ST_STEP);
  };
  // chunk i of the next Q tile (rows 8 i .. 8 i + 7 at d = 256) to LDS offset
  // base + i ST_STEP; for QSPLIT the caller passes the base of the chunk's half
  auto dma_qn = [&](int base, int i) __attribute__((always_inline)) {
    buf_load16_lds_off<PERSIST>(qrn, smem + (base + i * ST_STEP + dma_wave), st_ki(i),
                                q0n * C::ROWB, i * ST_STEP);
  };
  // bfloat16 V: the P V product runs in binary16, so each thread widens the chunks its
  // own loads wrote (chunk i: 16 bytes at dma_wave + i ST_STEP + 16 lane), in place.
  // Needs only this wave's loads to have landed; other waves read the stage after the
  // barrier that ends the iteration.
  auto widen_v = [&](char *vb, int i) __attribute__((always_inline)) {
    if constexpr (BF16) {
      char *p = vb + dma_wave + i * ST_STEP;
      u32x4 vv = lds_read16(p, lane * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) vv[q] = bf16x2_to_f16x2(vv[q]);
      lds_write16(p, lane * 16, vv);
    }
  };
  // the same in two parts, a few pipeline steps apart, so that the wave does not wait
  // for the read (and, LDS reads completing in order, for every operand read before it)
  u32x4 wv;
  auto widen_read = [&](char *vb, int i) __attribute__((always_inline)) {
    if constexpr (BF16) wv = lds_read16(vb + dma_wave + i * ST_STEP, lane * 16);
  };
  auto widen_write = [&](char *vb, int i) __attribute__((always_inline)) {
    if constexpr (BF16) {
      u32x4 vv = wv;
#pragma unroll
      for (int q = 0; q < 4; ++q) vv[q] = bf16x2_to_f16x2(vv[q]);
      lds_write16(vb + dma_wave + i * ST_STEP, lane * 16, vv);
    }
  };
  // operand of matrix-core step i: S^T step i = (block t = i / KC, k-step i % KC);
  // P V step i = (output block e = i % OB, key step u = i / OB).  kb / vb are the lane's
  // base offsets into the K / V stage being read (stage offset + k_base / v_base).
  // k_xor is a multiple of 32 below 256, so (32 kc) ^ k_xor = 256 (kc / 8) + ((32 (kc % 8))
  // ^ k_xor): eight absolute lane addresses per K stage (k_bases, once per tile), the rest
  // of an operand's address an immediate of its read
  constexpr int NKB = C::KC < 8 ? C::KC : 8;
  struct KBases {
    uint32_t c[NKB];
  };
  auto k_bases = [&](int kb) __attribute__((always_inline)) {
    KBases r;
#pragma unroll
    for (int e = 0; e < NKB; ++e) r.c[e] = lds_addr(smem) + uint32_t(kb + ((32 * e) ^ k_xor));
    return r;
  };
  auto k_op = [&](const KBases &kcb, int i) __attribute__((always_inline)) {
    const int t = i / C::KC, kc = i % C::KC;  // block-major: all k-steps of block 0 first
    return lds_read16_at(kcb.c[kc % 8] + 256 * (kc / 8) + 32 * t * C::ROWB);
  };
  // v_xor is a multiple of 64 below 256, so (64 e) ^ v_xor = 256 (e / 4) + ((64 (e % 4)) ^
  // v_xor): four absolute lane addresses per V stage (v_bases, once per tile), and every
  // other part of an operand's address is an immediate of its transposing reads
  struct VBases {
    uint32_t c[4];
  };
  auto v_bases = [&](int vb) __attribute__((always_inline)) {
    VBases r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r.c[e] = lds_addr(smem) + uint32_t(vb + ((64 * e) ^ v_xor));
    return r;
  };
  auto v_op = [&](const VBases &vc, int i) __attribute__((always_inline)) {
    const int u = i / OB, e = i % OB;
    const uint32_t a = vc.c[e % 4] + 256 * (e / 4) + (16 * u) * C::ROWB;
    const u32x2 a0 = lds_read_tr_at(a);
    const u32x2 a1 = lds_read_tr_at(a + 8 * C::ROWB);
    return u32x4{a0[0], a0[1], a1[0], a1[1]};
  };

  f32x16 o[RB][OB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int e = 0; e < OB; ++e) o[r][e] = f32x16{};
  // online-softmax state of the lane's query row in each block: running max (base-2
  // units), this lane's partial row sum, and, for the tile whose P is pending, its rescale
  // factor alpha and P row sum; lazy form only: the partial sums of P as rounded to
  // binary16 for the P V product (lp, and rp for the pending tile)
  // pq: the newest P value, added to rs one exponential later (the sum keeps score order,
  // and its add never follows the exponential that produced its operand)
  float mc[RB], l[RB], alpha[RB], rs[RB], pq[RB], lp[RB], rp[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    mc[r] = -INFINITY;
    l[r] = alpha[r] = rs[r] = pq[r] = lp[r] = rp[r] = 0.f;
  }
  const int nkt = (NK + C::BN - 1) / C::BN;
  const int nlast = NK - (nkt - 1) * C::BN;  // valid keys of the last tile, 1 .. BN

  // ---- the softmax of one tile is split across the two halves of an iteration ----
  // S^T holds 32 scores per lane and block: key block 0 (keys 0-31 of the tile,
  // registers s[r][0]) and key block 1 (keys 32-63, s[r][1]); score x is s[r][x/16][x%16].
  //   during B (the P V product of the previous tile): the row max over all 32 scores,
  //     the new running max and alpha, then P = 2^(c s - c m) for key block 0, which is
  //     packed into operand blocks 0 and 1 as soon as the previous tile's P V steps
  //     release them
  //   during A (the S product of the next tile, which rebuilds s[r][0] first and s[r][1]
  //     last): P for key block 1, packed into operand blocks 2 and 3 before s[r][1] is
  //     overwritten, the row sum, l = alpha l + sum, and O = alpha O
  // The row sum adds the 32 values of P in score order, as a single pass would.
  //
  // At d >= 128 (LAZY) the reference max mc moves only when a tile's row max exceeds it
  // by more than kTau (base-2 units): P <= 2^kTau stays far inside binary16 range,
  // softmax is unchanged by the choice of reference, and most tiles leave every alpha at
  // 1, so O is rescaled in a wave-uniform branch that is rarely taken instead of on every
  // tile.  That matters most where the output accumulators live in the matrix-core
  // (AGPR) registers (d = 256, two query blocks per wave at d = 128), where a multiply
  // costs a read, the multiply and a write per element; at d = 128 it saves 64
  // multiplies per tile (+1.5 % measured).  P > 1 then carries the binary16 rounding of values that are not
  // powers of two even for the row's largest score, so O is normalised by the sum of P
  // as rounded for the P V product (the weights applied to V sum to one) and LSE by the
  // exact sum.  At d = 64 the rescale every tile measured faster.
  constexpr bool LAZY = D >= 128;
  constexpr float kTau = RB == 2 ? 15.0f : 8.0f;
  constexpr int KC = C::KC;
  constexpr int NMX = NB >= 16 ? 2 : 1;  // B steps of the row max
  constexpr int NEB = NB - NMX - 1;      // B steps carrying key-block-0 exponentials
  constexpr int NEA = KC - 1;            // A steps carrying key-block-1 exponentials
  // S of the tile being started (becomes its P in place); the packed P of the tile
  // whose P V product is pending lives in pf
  f32x16 s[RB][SB];
  u32x4 pf[RB][PU];
  u32x4 kf[DK], vf[DV];
  float mx[RB], sub[RB];
  // Each step below acts on query block r alone: with two blocks per wave every
  // pipeline step is two sub-steps, one block's matrix-core product followed by that
  // block's share of the vector work, so that the vector work of one sub-step runs while
  // the product just issued occupies the matrix core.
  // With two query blocks per wave the second half of A carries no softmax work, so the
  // row max over key block 0 (complete after A step KC - 1) is taken there, on A steps
  // KC + 2 .. 2 KC - 1 (EARLY_MAX), and B takes only key block 1's.
  constexpr bool EARLY_MAX = RB == 2;
  // The P V products go through their own assembly into AGPR accumulators whenever O
  // cannot share the vector registers with S: two query blocks per wave at d = 128, or
  // d = 256 (O alone is 128 registers).  The unit is then compiled with the compiler's
  // own products (S) in vector-register form, so S is never copied out of AGPRs.  (Two
  // blocks at d = 64 keep everything in vector registers: 255-256 of them, two waves
  // per SIMD.)
  constexpr bool ASMPV = (RB == 2 && D > 64) || D == 256;
  constexpr int NAM = KC - 2;  // A steps carrying the key-block-0 max
  // the row max takes IEEE maximum, not fmaxf: the scores are finite or -inf, where the two
  // agree, and maximum needs no quieting of its operands (three-input v_maximum3_f32)
  auto max_range = [&](int b, int e, int r) __attribute__((always_inline)) {
    if (b == 0) mx[r] = s[r][0][0];
#pragma unroll
    for (int x = 0; x < 32; ++x)
      if (x >= b && x < e) mx[r] = __builtin_elementwise_maximum(mx[r], s[r][x / 16][x % 16]);
  };
  auto max_a = [&](int k, int r) __attribute__((always_inline)) {  // A step KC + 2 + k
    max_range(k * 16 / NAM, (k + 1) * 16 / NAM, r);
  };
  auto max_step = [&](int k, int r) __attribute__((always_inline)) {
    if constexpr (EARLY_MAX)
      max_range(16 + k * 16 / NMX, 16 + (k + 1) * 16 / NMX, r);
    else
      max_range(k * 32 / NMX, (k + 1) * 32 / NMX, r);
  };
  auto finalize_max = [&](int r) __attribute__((always_inline)) {
    const float m = pair_max(mx[r]);  // full row max over the tile's keys
    // running max in base-2 units (lazy: the reference, moved only past mc + kTau;
    // -inf + kTau stays -inf, so the first tile with a valid key always sets it)
    const float mxc = m * c;
    const float mc_new = LAZY ? (mxc > mc[r] + kTau ? mxc : mc[r])
                               : __builtin_elementwise_maximum(mc[r], mxc);
    // a row that has seen only masked keys keeps alpha = 0 and P = 0 (no inf - inf)
    alpha[r] = (mc[r] == -INFINITY) ? 0.f : ex2(mc[r] - mc_new);
    sub[r] = (mc_new == -INFINITY) ? 0.f : mc_new;
    mc[r] = mc_new;
    rs[r] = 0.f;
    pq[r] = 0.f;
    rp[r] = 0.f;
  };
  auto exp_range = [&](int b, int e, int r) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 32; ++x)
      if (x >= b && x < e) {
        const float p = ex2(fmaf(s[r][x / 16][x % 16], c, -sub[r]));
        s[r][x / 16][x % 16] = p;
        rs[r] += pq[r];
        pq[r] = p;
      }
  };
  // keys at or past nvalid of a tile are masked to -inf before its softmax
  auto mask_block = [&](int t, int nvalid) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int key = 32 * t + 8 * (x >> 2) + 4 * h + (x & 3);
        if (key >= nvalid) s[r][t][x] = -INFINITY;
      }
  };
  auto mask = [&](int nvalid) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < SB; ++t) mask_block(t, nvalid);
  };
  // P (fp32, S^T register layout) -> binary16 operands: step u takes key block u/2,
  // registers 8(u%2) .. +7, i.e. keys 16u + 8x + 4h + s for slot 4x + s
  auto pack_u = [&](int u, int r) __attribute__((always_inline)) {
    const int t = u >> 1, rb = (u & 1) * 8;
    pf[r][u] = u32x4{pack_f16(s[r][t][rb + 0], s[r][t][rb + 1]),
                     pack_f16(s[r][t][rb + 2], s[r][t][rb + 3]),
                     pack_f16(s[r][t][rb + 4], s[r][t][rb + 5]),
                     pack_f16(s[r][t][rb + 6], s[r][t][rb + 7])};
    pin(pf[r][u]);
    if constexpr (LAZY) rp[r] = sum8_f16(pf[r][u], rp[r]);
  };
  // B step k's share of the softmax; operand block u (0 or 1) is packed at the first
  // step where its 8 exponentials are done and its last reader (step OB u + OB - 1) of the
  // previous tile's P V product has issued
  auto b_exp_end = [](int k) __attribute__((always_inline)) {
    return k <= NMX ? 0 : (k - NMX) * 16 / NEB;
  };
  auto b_pack_step = [&](int u) __attribute__((always_inline)) {
    int k = NMX + 1;
    while (b_exp_end(k) < 8 * u + 8) ++k;
    return k > OB * u + OB ? k : OB * u + OB;
  };
  auto soft_b = [&](int k, int r) __attribute__((always_inline)) {
    if (k < NMX) max_step(k, r);
    else if (k == NMX) finalize_max(r);
    else exp_range(b_exp_end(k - 1), b_exp_end(k), r);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (b_pack_step(u) == k) pack_u(u, r);
  };
  // A step k's share: key-block-1 exponentials on steps 0 .. NEA-1, then (step NEA) the
  // last two operand blocks and l; O = alpha O on the steps that rebuild s[r][1]
  // statistics form: the tile whose softmax the next A half completes, and the record of
  // (c m, l) for block r once l includes it (both lanes of a row pair hold half of l)
  int st_tile = 0;
  auto record_stats = [&](int r) __attribute__((always_inline)) {
    const float lt = pair_sum(l[r]);
    const int row = q0 + 32 * (RB * w + r) + l32;
    if (h == 0 && row < N) {
      float *p = ST + ((int64_t(bh) * N + row) * nkt + st_tile) * 2;
      p[0] = mc[r];
      p[1] = lt;
    }
  };
  auto soft_a = [&](int k, int r, bool with_max = true) __attribute__((always_inline)) {
    if (k < NEA) exp_range(16 + k * 16 / NEA, 16 + (k + 1) * 16 / NEA, r);
    if (k == NEA) {
      pack_u(2, r);
      pack_u(3, r);
      rs[r] += pq[r];  // the tile's last P value
      l[r] = fmaf(l[r], alpha[r], rs[r]);
      if constexpr (LAZY) lp[r] = fmaf(lp[r], alpha[r], rp[r]);
      if constexpr (STATS) record_stats(r);
    }
    if (EARLY_MAX && with_max && k >= KC + 2) max_a(k - KC - 2, r);
    if (!LAZY && k >= KC) {
      constexpr int R = OB * 16 / KC;
      const int q = k - KC;
#pragma unroll
      for (int x = 0; x < OB * 16; ++x)
        if (x >= q * R && x < (q + 1) * R) o[r][x / 16][x % 16] *= alpha[r];
      pin(o[r][q * R / 16]);
    }
  };

  // lazy form: O = alpha O for the whole tile, skipped when every alpha of the wave is 1
  auto rescale_lazy = [&]() __attribute__((always_inline)) {
    if constexpr (LAZY) {
      bool any = false;
#pragma unroll
      for (int r = 0; r < RB; ++r) any |= alpha[r] != 1.0f;
      if (__builtin_amdgcn_ballot_w64(any) != 0) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int e = 0; e < OB; ++e) {
#pragma unroll
            for (int x = 0; x < 16; ++x) o[r][e][x] *= alpha[r];
            if constexpr (RB == 2) __builtin_amdgcn_sched_barrier(0);  // a block at a time
          }
      }
    }
  };

  // S product step i of block r, block-major so s[r][0] is rebuilt before s[r][1]; one
  // K operand feeds every query block of the wave
  auto s_step = [&](int i, u32x4 kop, int r) __attribute__((always_inline)) {
    const int t = i / KC, kc = i % KC;
    s[r][t] = mma16<BF16>(kop, qf[r][kc], kc == 0 ? f32x16{} : s[r][t]);
  };
  // after the last P V product of a phase: wait for the products to finish, then give O
  // fresh definitions there, so that every later read of the accumulators (the lazy
  // rescale, copies the compiler makes, the epilogue) follows the wait
  auto settle_o = [&]() __attribute__((always_inline)) {
    if constexpr (ASMPV) {
      mfma_drain();
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int e = 0; e < OB; ++e) asm volatile("" : "+a"(o[r][e]));
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // P V product step i of block r: one V operand feeds every query block of the wave
  auto pv_step = [&](int i, u32x4 vop, int r) __attribute__((always_inline)) {
    const int u = i / OB, e = i % OB;
    if constexpr (ASMPV)
      asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                   : "+a"(o[r][e])
                   : "v"(vop), "v"(pf[r][u]));
    else
      o[r][e] = mma_f16(vop, pf[r][u], o[r][e]);
  };

  // Loads into LDS are waited for explicitly: each wave waits (s_waitcnt vmcnt, loads
  // retire in issue order) for its own loads of the stages the next barrier publishes,
  // and leaves the younger ones in flight.
  auto wait_loads = [](auto n) __attribute__((always_inline)) {  // at most n.value of this wave's loads in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_only(decltype(n)::value));
  };
  using in_flight_0 = std::integral_constant<int, 0>;
  using in_flight_1 = std::integral_constant<int, CPT>;  // one tile of K or V

  // ---- prologue: K_0, V_0 and K_1 staged; S_0 and the B share of its softmax ----
  dma_k(Ks, 0);
  dma_v(Vs, 0);
  dma_k(Ks + C::TILEB, 1);
  // K_0 and V_0 have landed (persistent form: K_1 too, as for every later tile)
  if constexpr (PERSIST)
    wait_loads(in_flight_0{});
  else
    wait_loads(in_flight_1{});
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) widen_v(Vs, i);
  }
  lds_barrier();
  // LDS stage of the tile's K_0 and V_0: K_j and V_j sit in stage (j + sb) % 2.  In the
  // persistent form the stages alternate across tiles as if their key tiles were one
  // sequence, so that the next tile's first tiles go to the stages the current tile's
  // last ones have left.
  int sb = 0;
  static_assert(!PERSIST || (RB == 1 && (D == 128 || D == 256)),
                "persistent form: one 32-row block per wave, d = 128 or 256");
  for (;;) {
    const KBases kc0 = k_bases(k_base + sb * C::TILEB);
#pragma unroll
    for (int i = 0; i < DK; ++i) kf[i] = k_op(kc0, i);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
#pragma unroll
      for (int r = 0; r < RB; ++r) s_step(i, kf[i % DK], r);
      if (i + DK < NA) kf[i % DK] = k_op(kc0, i + DK);
      __builtin_amdgcn_sched_barrier(0);  // the reads stay DK steps ahead of their products
    }
    if (nkt == 1 && nlast < C::BN) mask(nlast);
    if constexpr (EARLY_MAX) {
#pragma unroll
      for (int k = 0; k < NAM; ++k)
#pragma unroll
        for (int r = 0; r < RB; ++r) max_a(k, r);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
#pragma unroll
      for (int r = 0; r < RB; ++r) soft_b(k, r);
      __builtin_amdgcn_sched_barrier(0);
    }
    // K_1 has landed, and every wave is done with K_0 before its stage is refilled
    // (persistent form at d = 128: K_1 landed before the previous barrier; at d = 256 it was
    // issued after the previous tile's Q left its K stage)
    if constexpr (!PERSIST || QSPLIT) wait_loads(in_flight_0{});
    lds_barrier();

    // ---- steady state: iteration j (P = (j + sb) % 2 selects the LDS stages) ----
    //   A: V_{j+1} and K_{j+2} start towards LDS; S_{j+1} = K_{j+1} Q^T on the matrix
    //      cores, while the VALU finishes the softmax of tile j and rescales O by alpha_j
    //   B: O += V_j P_j on the matrix cores, while the VALU starts the softmax of S_{j+1}
    //      and widens bfloat16 V_{j+1}
    // The stages written in iteration j held K_j and V_{j-1}, last read in iteration j-1;
    // the barrier that ends each iteration orders every stage's last read before its next
    // write, and every write before its next read: before it each wave waits for its
    // loads of V_{j+1} and K_{j+2}, which iteration j + 1 reads.  B waits for V_{j+1}
    // alone (it was issued first) before widening it, and the transposing reads of V_j
    // wait for nothing.
    // MASKED: the tile started in this iteration (j + 1) is the last one, so its keys past
    // N are masked; only the final iteration is compiled with it, keeping the mask out of
    // the steady-state loop.  In the persistent form that iteration loads the next tile's
    // K_0 in place of K_{j+2} (past the end), then the next tile's Q, which its waits leave
    // in flight.
    auto iter = [&](int j, auto masked) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked)::value;
      constexpr bool NEXT = PERSIST && MASKED;
      constexpr int QSTEPS = NA - 2 * CPT;  // A steps that carry the next tile's Q
      // first A step of K_{j+2}'s loads: at d = 128 and 256 in the second half of A, whose
      // steps carry no softmax work, instead of right after V_{j+1}'s (measured: d = 256
      // +5.1 %, c3 +1.4 %; bitwise the same)
      constexpr int K0 = ((D == 256 || D == 128) && !NEXT) ? NA / 2 : CPT;
      // chunks of the next Q issued here (QSPLIT: the half bound for Xs)
      constexpr int QIN = QSPLIT ? C::QCPT / 2 : C::QCPT;
      static_assert(!NEXT || QSTEPS >= 1, "the next tile's Q needs A steps of its own");
      const int P = (j + sb) & 1;
      // lane bases of this iteration's reads (the pins keep the offset arithmetic inside
      // the loop rather than precomputed into live registers)
      pin(k_xor);
      pin(v_xor);
      const int kb = k_base + (1 - P) * C::TILEB;         // K_{j+1}
      const int vb = v_base + (2 + P) * C::TILEB;         // V_j
      char *vw = Vs + (1 - P) * C::TILEB;                 // V_{j+1}, widened in B
      char *kw = Ks + P * C::TILEB;                       // K_{j+2}

      // ---- A ----
      // (one wait for the operands of two consecutive products, PAIRW: with one query block
      // per wave each product would otherwise wait for its own; the compiler's waits stay
      // and find these already met)
      st_tile = j;
      rescale_lazy();
      const KBases kcb = k_bases(kb);
#pragma unroll
      for (int i = 0; i < DK; ++i) kf[i] = k_op(kcb, i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          // K reads of steps i + 2 .. min(i + DK, NA) - 1 may stay in flight
          if (PAIRW && r == 0 && i % 2 == 0 && i + 1 < NA) {
            wait_lds(imin(DK - 2, NA - i - 2));
            __builtin_amdgcn_sched_barrier(0);  // the products stay behind the wait
          }
          s_step(i, kf[i % DK], r);
          if (r == RB - 1 && i + DK < NA) kf[i % DK] = k_op(kcb, i + DK);
          // V_{j+1} first (B waits for it alone), then K_{j+2}
          if (r == 0 && i < CPT) dma_v1(vw, j + 1, i, std::integral_constant<bool, NEXT>{});
          if (r == 0 && i >= K0 && i < K0 + CPT) {
            if constexpr (NEXT)
              dma_kn(kw, 0, i - K0);
            else
              dma_k1(kw, j + 2, i - K0, std::false_type{});
          }
          if constexpr (NEXT) {
#pragma unroll
            for (int q = 0; q < QIN; ++q)
              if (r == 0 && i >= 2 * CPT && q * QSTEPS / QIN == i - 2 * CPT)
                dma_qn(QSPLIT ? XS_OFF : int(Qs - smem), q);
          }
          // the last tile's keys past N are masked before its early max reads key block 0
          if (EARLY_MAX && MASKED && i == KC + 1 && r == 0 && nlast < C::BN)
            mask_block(0, nlast);
          soft_a(i, r);
          __builtin_amdgcn_sched_barrier(0);
        }

      // ---- B ----
      const VBases vc = v_bases(vb);
#pragma unroll
      for (int i = 0; i < DV; ++i) vf[i] = v_op(vc, i);
      if (MASKED && nlast < C::BN) mask(nlast);
      // bfloat16 V_{j+1} is widened in place during the P V product below, once this
      // wave's loads of it have landed (the loads issued after it may stay in flight)
      if constexpr (BF16) {
        if constexpr (NEXT)
          wait_loads(std::integral_constant<int, CPT + QIN>{});
        else
          wait_loads(in_flight_1{});
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          // V reads of steps i + 2 .. min(i + DV, NB) - 1 (two each) and the widening's LDS
          // accesses of the steps since then may stay in flight
          if (PAIRW && r == 0 && i % 2 == 0 && i + 1 < NB) {
            wait_lds(2 * imin(DV - 2, NB - i - 2) + widen_ops(i + 2 - DV, i));
            __builtin_amdgcn_sched_barrier(0);
          }
          pv_step(i, vf[i % DV], r);
          if (r == RB - 1 && i + DV < NB) vf[i % DV] = v_op(vc, i + DV);
          soft_b(i, r);
          {
            // chunk c: read at step (NB / CPT) c + 1, widened and written back at the
            // chunk's last step
            if (r == 0 && i % (NB / CPT) == 1) widen_read(vw, i / (NB / CPT));
            if (r == RB - 1 && i % (NB / CPT) == NB / CPT - 1) widen_write(vw, i / (NB / CPT));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      settle_o();
      if constexpr (NEXT)
        wait_loads(std::integral_constant<int, QIN>{});  // the next tile's Q may fly on
      else
        wait_loads(in_flight_0{});
      lds_barrier();
    };

    for (int j = 0; j + 2 < nkt; ++j) iter(j, std::false_type{});
    if constexpr (PERSIST) set_next();  // (here, so that its registers are not held in the loop)
    if (nkt >= 2) iter(nkt - 2, std::true_type{});

    // ---- last tile T = nkt - 1: the A share of its softmax, then its P V product ----
    // (persistent form: the next tile's V_0 goes to the stage V_{T-1} has left, and its K_1
    // (d = 128) or the second half of its Q (d = 256) to the stage K_T has left)
    const int sbn = (sb + nkt) & 1;  // the next tile's stage base
    // QSPLIT: LDS offset of the next Q's row 0 for its second half (rows BM/2 .. in the K
    // stage K_T has left)
    const int qhi = (1 - sbn) * C::TILEB - (C::QCPT / 2) * ST_STEP;
    {
      if constexpr (PERSIST) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) dma_vn(Vs + sbn * C::TILEB, 0, i);
        if constexpr (QSPLIT) {
#pragma unroll
          for (int q = C::QCPT / 2; q < C::QCPT; ++q) dma_qn(qhi, q);
        } else {
#pragma unroll
          for (int i = 0; i < CPT; ++i) dma_kn(Ks + (1 - sbn) * C::TILEB, 1, i);
        }
      }
      const VBases vc = v_bases(v_base + (2 + ((nkt - 1 + sb) & 1)) * C::TILEB);
      st_tile = nkt - 1;
      rescale_lazy();
#pragma unroll
      for (int k = 0; k < NA; ++k)
#pragma unroll
        for (int r = 0; r < RB; ++r) soft_a(k, r, false);
      if constexpr (ASMPV) mfma_drain();
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const u32x4 vop = v_op(vc, i);
#pragma unroll
        for (int r = 0; r < RB; ++r) pv_step(i, vop, r);
      }
      settle_o();
    }

    if constexpr (PERSIST) {
      // the next tile's Q, K_0, V_0 (and at d = 128 K_1) have landed; this thread widens
      // its own chunks of V_0, then (after the barrier) every wave takes its Q rows, and
      // after a second barrier the Q region holds the output on its way out
      wait_loads(in_flight_0{});
      if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) widen_v(Vs + sbn * C::TILEB, i);
      }
      lds_barrier();
      if (has_next) {
        if constexpr (QSPLIT)
          read_q(32 * w < C::BM / 2 ? XS_OFF : qhi);
        else
          read_q(int(Qs - smem));
      }
    }
    // every wave is done with the LDS region that holds the output (the K/V stages, or in
    // the persistent form the Q region; QSPLIT: Xs and the V stage V_T has left)
    lds_barrier();
    if constexpr (QSPLIT) {
      // the next tile's K_1, to the K stage the second half of its Q has left (only if
      // there is one: nothing may still be loading into LDS when the workgroup ends)
      if (has_next) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) dma_kn(Ks + (1 - sbn) * C::TILEB, 1, i);
      }
    }
    // bytes of a wave's region (QSPLIT: two waves' regions in each 32 KiB half)
    constexpr int WAVE_LDS = (PERSIST ? C::QB : C::LDS) / WAVES;
    constexpr int NHALF = (32 * D * 4 + WAVE_LDS - 1) / WAVE_LDS;
    // QSPLIT: waves 0 .. WAVES/2-1 stage in Xs, the others in the V stage V_T has left
    const int out_off = !QSPLIT ? int(Qs - smem) + w * WAVE_LDS
                        : w < WAVES / 2 ? XS_OFF + w * WAVE_LDS
                                        : 2 * C::TILEB + (1 - sbn) * C::TILEB +
                                              (w - WAVES / 2) * WAVE_LDS;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row0 = q0 + 32 * (RB * w + r);  // the block's first query row
      store_rows_lds<D, NHALF>(o[r], mc[r], l[r], LAZY ? lp[r] : l[r], smem + out_off,
                               O + kg * bhn * D + hoff + int64_t(row0) * D,
                               LSE + kg * bhn + int64_t(bh) * N + row0, lane, N - row0);
    }
    if (!PERSIST || !has_next) break;

    // ---- the next tile: fresh online-softmax state and output accumulators ----
    vt += gridDim.x;
    set_tile(vt);
    sb = sbn;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
#pragma unroll
      for (int e = 0; e < OB; ++e) o[r][e] = f32x16{};
      mc[r] = -INFINITY;
      l[r] = alpha[r] = rs[r] = pq[r] = lp[r] = rp[r] = 0.f;
    }
  }
}

// Launch of the 16-bit kernel with WAVES waves of RB 32-row query blocks each.
// nsplit key ranges of kps keys each (the last may be shorter, none is empty); with
// nsplit = 1 and kps = N the kernel writes the attention itself to o and lse
// STATS: the statistics-recording form, writing to stats (nsplit = 1).
// With nsplit = 1, at least two key tiles, d = 128 or 256 and more tiles than the device holds
// workgroups at once, the persistent form runs instead: one workgroup per resident slot,
// each taking its tiles in turn.
template <int D, bool BF16, int WAVES, int RB, bool STATS = false>
inline hipError_t run16(const Problem &p, float *o, float *lse, int nsplit, int kps,
                        hipStream_t stream, float *stats = nullptr) {
  using C = Cfg16<D, WAVES, RB>;
  const int nqt = (p.N + C::BM - 1) / C::BM;
  const int G = nqt * p.B * p.H * nsplit;
  const float c = p.scale * kLog2e;
  if constexpr (!STATS && (D == 128 || D == 256)) {
    if (nsplit == 1 && p.N > C::BN) {
      constexpr auto pk = fa_fwd16_kernel<D, BF16, WAVES, RB, false, true>;
      const int R = resident_workgroups<pk>(C::NT, C::LDSP);
      if (R >= 8 && G > R) {
        const hipError_t ea = allow_lds_on_device<pk>(C::LDSP);
        if (ea != hipSuccess) return ea;
        // a multiple of 8, so that workgroup b keeps the XCD (b mod 8) of all its tiles
        hipLaunchKernelGGL(pk, dim3(R & ~7), dim3(C::NT), C::LDSP, stream,
                           static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.k),
                           static_cast<const uint16_t *>(p.v), o, lse, p.N, nqt, G, c, 1, p.N,
                           stats);
        return hipGetLastError();
      }
    }
  }
  auto kern = fa_fwd16_kernel<D, BF16, WAVES, RB, STATS>;
  const hipError_t ea =
      allow_lds_on_device<fa_fwd16_kernel<D, BF16, WAVES, RB, STATS>>(C::LDS);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL(kern, dim3(G), dim3(C::NT), C::LDS, stream,
                     static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.k),
                     static_cast<const uint16_t *>(p.v), o, lse, p.N, nqt, G, c, nsplit, kps,
                     stats);
  return hipGetLastError();
}

}  // namespace fa
