// Device-side building blocks for the gfx950 attention kernels: vector types,
// matrix-core wrappers, LDS address swizzles and lane exchanges.
//
// Register layouts used throughout (checked against exact integer products on
// gfx950; "lane" is the lane id 0..63, "h" = lane / 32):
//   v_mfma_f32_32x32x16_{bf16,f16}  A[32 x 16]: lane holds A[lane % 32][8h .. 8h+7]
//                                   B[16 x 32]: lane holds B[8h .. 8h+7][lane % 32]
//                                   C[32 x 32]: register r of lane holds
//                                     C[8*(r/4) + 4h + r%4][lane % 32]
//   v_mfma_f32_32x32x2_f32          A: lane holds A[lane % 32][h], B: B[h][lane % 32],
//                                   C as above.
//   ds_read_b64_tr_b16              within each group of 16 lanes, lane i receives, for
//                                   s = 0..3, element (i % 4) of the four 16-bit values
//                                   addressed by lane 4s + i/4 of its group.
//   v_permlane32_swap               exchanges a register between lane l and lane l ^ 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- matrix cores ---------------------------------------------------------------
__device__ __forceinline__ f32x16 mma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <bool BF16>
__device__ __forceinline__ f32x16 mma16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16)
    return mma_bf16(a, b, c);
  else
    return mma_f16(a, b, c);
}
__device__ __forceinline__ f32x16 mma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Matrix-core products written as assembly (accumulating in AGPRs) are not tracked by
// the compiler's hazard recognizer: vector code that reads their accumulators must first
// wait for the last product explicitly.  24 wait states, more than the 19 of the longest
// (16-pass) product; the fences keep the wait where it is placed.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ---- lane exchange --------------------------------------------------------------
// v_permlane32_swap(a, b) swaps the upper 32 lanes of a with the lower 32 lanes of b.
// With a = b = x the two results hold, on every lane l, x[min(l, l^32)] and
// x[max(l, l^32)]: the lane's own value and its partner's, in the same order on
// both lanes of a pair, so the combined value below is bitwise equal on both.
__device__ __forceinline__ void pair_values(float x, float &lo, float &hi) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  lo = __builtin_bit_cast(float, (uint32_t)p[0]);
  hi = __builtin_bit_cast(float, (uint32_t)p[1]);
}
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  pair_values(x, a, b);
  return __builtin_elementwise_maximum(a, b);  // (finite or -inf operands: as fmaxf)
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  pair_values(x, a, b);
  return a + b;
}

// ---- fast math ---------------------------------------------------------------------
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ---- conversions -----------------------------------------------------------------
// two fp32 -> packed binary16, round to nearest even
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// two packed bfloat16 -> two packed binary16 (exact for normal binary16 range)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  float lo = __builtin_bit_cast(float, w << 16);
  float hi = __builtin_bit_cast(float, w & 0xffff0000u);
  return pack_f16(lo, hi);
}

// sum of the eight binary16 values packed in v, added to acc in fp32 (each product by 1
// is exact; v_dot2_f32_f16 accumulates in fp32)
__device__ __forceinline__ float sum8_f16(u32x4 v, float acc) {
  const f16x8 x = __builtin_bit_cast(f16x8, v);
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  acc = __builtin_amdgcn_fdot2(f16x2{x[0], x[1]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2(f16x2{x[2], x[3]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2(f16x2{x[4], x[5]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2(f16x2{x[6], x[7]}, one, acc, false);
  return acc;
}

// ---- LDS swizzles (units: 16-byte chunks; cpr = chunks per row) -------------------
// Row-operand tiles (Q, K) are read 16 bytes per lane with 16 lanes on 16
// consecutive rows at the same logical chunk: spread those 16 rows over all banks.
template <int CPR>
__device__ __forceinline__ int swz_row(int r, int ch) {
  if constexpr (CPR == 8)
    return ch ^ ((r >> 1) & 7);
  else
    return ch ^ (r & 15);
}
// V tiles are read with the transposing load: 8 consecutive rows, each reading one
// 64-byte block (4 chunks).  Rotate the 64-byte blocks so 4 consecutive rows cover
// all 256 bytes of the bank space.
template <int CPR>
__device__ __forceinline__ int swz_v(int r, int ch) {
  if constexpr (CPR == 8)
    return ch ^ (((r >> 1) & 1) << 2);
  else
    return ch ^ ((r & 3) << 2);
}

// ---- bounds-checked global loads ----------------------------------------------------
// A raw buffer resource over `bytes` bytes from `base`: 16-byte loads whose byte offset
// (VGPR offset + SGPR offset, both range-checked on gfx950) is at or beyond `bytes`
// return zeros without touching memory, which pads the ragged last tile of a head.
// The third resource word selects 32-bit elements (gfx9 family).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// 16 bytes per lane from global memory straight into LDS, without passing through
// registers: lane l of the wave writes lds_wave_base + 16 l (lds_wave_base is uniform
// across the wave; m0 carries it, and one wait state separates its write from the load).
// Out-of-range dwords are written as zeros.  Completion is counted by vmcnt like any
// other global load, in issue order.
//
// The load is issued as inline assembly, which the compiler's wait-count tracking does
// not see.  For the builtin form the compiler cannot tell which LDS stage a later
// transposing read addresses, so it waits for every load into LDS in flight before each
// such read, including loads of stages read only in later iterations.  Here the caller
// waits explicitly (s_waitcnt vmcnt) for exactly the loads a barrier publishes.  The
// compiler's own waits for the loads it tracks stay correct: loads retire in order, so
// extra untracked loads can only make those waits longer.
//
// Nor does the compiler keep, before inline assembly, the 5 wait states a vector-memory
// instruction needs after a vector instruction writes one of its scalar operands (a
// scalar restored from a spill with v_readlane, for instance).  SAFE = true puts them in
// front of the load, for kernels whose scalar registers spill; the assembly hazard test
// checks every kernel for both forms.
template <bool SAFE = false>
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, char *lds_wave_base,
                                               int voff, int soff) {
  const uint32_t m0v =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds_wave_base;
  if constexpr (SAFE)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(soff), "{m0}"(m0v)
                 : "memory");
  else
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(soff), "{m0}"(m0v)
                 : "memory");
}

// The same load with its scalar offset soff_base + soff_imm, soff_imm a constant once
// loops are unrolled: the add runs inside the assembly, in front of the load, where it
// also stands in the one wait state after the m0 write (SAFE: it and s_nop 3 give 5).
template <bool SAFE = false>
__device__ __forceinline__ void buf_load16_lds_off(__amdgpu_buffer_rsrc_t r, char *lds_wave_base,
                                                   int voff, int soff_base, int soff_imm) {
  const uint32_t m0v =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds_wave_base;
  int so;
  if constexpr (SAFE)
    asm volatile("s_add_i32 %0, %2, %4\n\ts_nop 3\n\tbuffer_load_dwordx4 %1, %3, %0 offen lds"
                 : "=&s"(so)
                 : "v"(voff), "s"(soff_base), "s"(r), "i"(soff_imm), "{m0}"(m0v)
                 : "memory", "scc");
  else
    asm volatile("s_add_i32 %0, %2, %4\n\tbuffer_load_dwordx4 %1, %3, %0 offen lds"
                 : "=&s"(so)
                 : "v"(voff), "s"(soff_base), "s"(r), "i"(soff_imm), "{m0}"(m0v)
                 : "memory", "scc");
}

// Workgroup barrier that orders LDS accesses only: the loads into LDS above are not
// waited for here (the caller's s_waitcnt vmcnt decides which must have landed).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ u32x4 lds_read16(const char *base, int byte_off) {
  return *reinterpret_cast<const u32x4 *>(base + byte_off);
}
__device__ __forceinline__ void lds_write16(char *base, int byte_off, u32x4 v) {
  *reinterpret_cast<u32x4 *>(base + byte_off) = v;
}
__device__ __forceinline__ u32x2 lds_read_tr(const char *base, int byte_off) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + byte_off));
  return __builtin_bit_cast(u32x2, r);
}

// LDS reads from an absolute 32-bit LDS byte address.  A dynamic-LDS array's own
// address is a link-time constant that the compiler adds to every offset with a VALU add;
// folding it into a lane's address once leaves only immediate offsets at the reads.
typedef __attribute__((address_space(3))) char lds_byte;
__device__ __forceinline__ uint32_t lds_addr(const char *p) {
  return uint32_t(uintptr_t((const lds_byte *)p));
}
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
__device__ __forceinline__ u32x4 lds_read16_at(uint32_t addr) {
  return *(const lds_u32x4 *)(uintptr_t)addr;
}
__device__ __forceinline__ u32x2 lds_read_tr_at(uint32_t addr) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2, r);
}

// s_waitcnt immediate that waits for at most n outstanding vector-memory operations and
// leaves the other counters alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8)
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// the same for LDS operations (lgkmcnt), leaving vmcnt and expcnt alone
constexpr int lgkmcnt_only(int n) { return 15 | (3 << 14) | (7 << 4) | ((n & 15) << 8); }
// s_waitcnt lgkmcnt(n) for an n that is a constant once loops are unrolled (the builtin
// takes only constant expressions; the switch folds away)
__device__ __forceinline__ void wait_lds(int n) {
  switch (n) {
#define FA_WAIT_LDS(k) \
  case k:              \
    __builtin_amdgcn_s_waitcnt(lgkmcnt_only(k)); \
    break;
    FA_WAIT_LDS(0) FA_WAIT_LDS(1) FA_WAIT_LDS(2) FA_WAIT_LDS(3) FA_WAIT_LDS(4)
    FA_WAIT_LDS(5) FA_WAIT_LDS(6) FA_WAIT_LDS(7) FA_WAIT_LDS(8) FA_WAIT_LDS(9)
    FA_WAIT_LDS(10) FA_WAIT_LDS(11) FA_WAIT_LDS(12) FA_WAIT_LDS(13) FA_WAIT_LDS(14)
#undef FA_WAIT_LDS
    default:
      break;
  }
}

// ---- schedule pins ----------------------------------------------------------------
// An empty asm that claims to rewrite x: the value must be computed before this point
// and cannot be sunk past it, which keeps arithmetic in the pipeline step it was
// written in (the scheduler fences keep the steps themselves in order).
template <typename T>
__device__ __forceinline__ void pin(T &x) {
  asm volatile("" : "+v"(x));
}

// ---- workgroup order ----------------------------------------------------------------
// Workgroups are handed to the 8 XCDs round-robin (id % 8).  Renumber them so that
// consecutive logical ids - the Q tiles of one head, which read the same K/V -
// run on one XCD and share its L2.  Bijective for any grid size G.
__device__ __forceinline__ int xcd_remap(int w, int G) {
  int per = G >> 3, rem = G & 7;
  int x = w & 7, idx = w >> 3;
  return x * per + (x < rem ? x : rem) + idx;
}

}  // namespace fa
