// C boundary of libfa.so: argument checks, then one launch sequence on the caller's
// stream.  The contract of every entry point is documented in include/fa.h.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <limits>

#include "fa_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int elem_bytes(int dtype) { return dtype == FA_F32 ? 4 : 2; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Checks shared by both paths.  Sets *empty when there is nothing to compute.
int check_args(const void *q, const void *k, const void *v, const float *o, const float *lse,
               int B, int H, int N, int d, float scale, int dtype, bool *empty) {
  *empty = false;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  // index limits: B*H heads must fit an int, the grid must stay within kMaxGrid
  const int64_t heads = int64_t(B) * H;
  if (heads > std::numeric_limits<int>::max()) return FA_ERR_SHAPE;
  const int64_t qtiles = (int64_t(N) + fa::kFusedBM - 1) / fa::kFusedBM;
  if (heads * qtiles > fa::kMaxGrid) return FA_ERR_SHAPE;
  // one head's [N, d] slice is addressed with 32-bit byte offsets (plus one tile)
  if (int64_t(N) * d * elem_bytes(dtype) > fa::kMaxHeadBytes) return FA_ERR_SHAPE;
  return FA_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  g_last_hip_error = int(e);
  return FA_ERR_HIP;
}

int device_ready() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  return FA_OK;
}

fa::Problem make_problem(const void *q, const void *k, const void *v, float *o, float *lse,
                         int B, int H, int N, int d, float scale, int dtype) {
  fa::Problem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.dtype = dtype;
  return p;
}

}  // namespace

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, float *o, float *lse, int B, int H, int N,
           int d, float scale, int dtype, void *stream) {
  bool empty = false;
  int rc = check_args(q, k, v, o, lse, B, H, N, d, scale, dtype, &empty);
  if (rc != FA_OK || empty) return rc;
  rc = device_ready();
  if (rc != FA_OK) return rc;
  return hip_status(fa::launch_fused(make_problem(q, k, v, o, lse, B, H, N, d, scale, dtype),
                                     static_cast<hipStream_t>(stream)));
}

size_t fa_fwd_stats_bytes(int B, int H, int N) {
  if (B < 0 || H < 0 || N < 0) return 0;
  const unsigned __int128 n = (unsigned __int128)(uint64_t)B * (uint64_t)H * (uint64_t)N *
                              (uint64_t)((N + 63) / 64) * 2 * sizeof(float);
  if (n > (unsigned __int128)std::numeric_limits<size_t>::max())
    return std::numeric_limits<size_t>::max();
  return (size_t)n;
}

int fa_fwd_stats(const void *q, const void *k, const void *v, float *o, float *lse,
                 float *stats, int B, int H, int N, int d, float scale, int dtype, void *stream) {
  bool empty = false;
  int rc = check_args(q, k, v, o, lse, B, H, N, d, scale, dtype, &empty);
  if (rc != FA_OK || empty) return rc;
  if (!stats || !aligned(stats, 16)) return FA_ERR_WORKSPACE;
  if (fa_fwd_stats_bytes(B, H, N) == std::numeric_limits<size_t>::max()) return FA_ERR_SHAPE;
  rc = device_ready();
  if (rc != FA_OK) return rc;
  return hip_status(fa::launch_fused_stats(make_problem(q, k, v, o, lse, B, H, N, d, scale, dtype),
                                           stats, static_cast<hipStream_t>(stream)));
}

// Workspace of the key-split forward: nsplit slots of partial O (B H N d floats), then
// nsplit slots of partial LSE (B H N floats), each part starting on a 256-byte boundary.
namespace {
struct SplitLayout {
  unsigned __int128 lse, total;
};
SplitLayout split_layout(int B, int H, int N, int d, int nsplit) {
  const unsigned __int128 rows =
      (unsigned __int128)(uint64_t)B * (uint64_t)H * (uint64_t)N * (uint64_t)nsplit;
  SplitLayout L;
  L.lse = (rows * (uint64_t)d * 4 + 255) / 256 * 256;
  L.total = L.lse + (rows * 4 + 255) / 256 * 256;
  return L;
}
}  // namespace

int fa_fwd_split_suggest(int B, int H, int N, int d, int compute_units) {
  if (B <= 0 || H <= 0 || N <= 0 || compute_units <= 0) return 1;
  if (d != 64 && d != 128 && d != 256) return 1;
  const int64_t rows_per_wg = d == 128 ? 256 : 128;  // query rows per fused workgroup
  const int64_t wgs = int64_t(B) * H * ((N + rows_per_wg - 1) / rows_per_wg);
  if (wgs >= compute_units) return 1;
  const int64_t want = (compute_units + wgs - 1) / wgs;
  const int64_t cap = std::max<int64_t>(1, ((N + 63) / 64) / 8);  // >= 8 key tiles per range
  return int(std::min<int64_t>({want, cap, int64_t(FA_MAX_SPLIT)}));
}

size_t fa_fwd_split_workspace_bytes(int B, int H, int N, int d, int nsplit) {
  if (B < 0 || H < 0 || N < 0 || nsplit < 1 || nsplit > FA_MAX_SPLIT) return 0;
  if (d != 64 && d != 128 && d != 256) return 0;
  const unsigned __int128 t = split_layout(B, H, N, d, nsplit).total;
  if (t > (unsigned __int128)std::numeric_limits<size_t>::max())
    return std::numeric_limits<size_t>::max();
  return (size_t)t;
}

}  // extern "C"

namespace {
// Checks of fa_fwd_split other than its workspace; *empty: nothing to compute.  Gives
// the ranges: kps keys each (whole 64-key tiles), `used` of them (ranges that would
// start past N are dropped).
int split_check(const void *q, const void *k, const void *v, const float *o, const float *lse,
                int nsplit, int B, int H, int N, int d, float scale, int dtype, bool *empty,
                int *kps, int *used) {
  int rc = check_args(q, k, v, o, lse, B, H, N, d, scale, dtype, empty);
  if (rc != FA_OK) return rc;
  if (nsplit < 1 || nsplit > FA_MAX_SPLIT) return FA_ERR_SHAPE;
  if (*empty) return FA_OK;
  const int tiles = (N + 63) / 64;
  *kps = (tiles + nsplit - 1) / nsplit * 64;
  *used = (N + *kps - 1) / *kps;
  const int64_t qtiles = (int64_t(N) + fa::kFusedBM - 1) / fa::kFusedBM;
  if (int64_t(B) * H * qtiles * *used > fa::kMaxGrid) return FA_ERR_SHAPE;
  return FA_OK;
}

int split_launch(const void *q, const void *k, const void *v, float *o, float *lse, char *ws,
                 int nsplit, int B, int H, int N, int d, float scale, int dtype, int kps,
                 int used, void *stream) {
  const SplitLayout L = split_layout(B, H, N, d, nsplit);
  return hip_status(fa::launch_fused_split(
      make_problem(q, k, v, o, lse, B, H, N, d, scale, dtype), reinterpret_cast<float *>(ws),
      reinterpret_cast<float *>(ws + (size_t)L.lse), used, kps, static_cast<hipStream_t>(stream)));
}
}  // namespace

// The allocation-free key split's scratch: FA_SCRATCH_BYTES of device memory per
// device, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory; the device address of each device's copy comes from
// hipGetSymbolAddress and is kept per device.
static __device__ __align__(256) unsigned char scratch[FA_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void *> g_scratch_addr[kScratchDevices];  // per device id; null until looked up

// This device's scratch address (looked up once per device, with the device current).
int scratch_address(void **addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  const bool cached = dev >= 0 && dev < kScratchDevices;
  void *p = cached ? g_scratch_addr[dev].load(std::memory_order_acquire) : nullptr;
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr) return FA_ERR_HIP;
    if (cached) g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *addr = p;
  return FA_OK;
}
}  // namespace

extern "C" {

int fa_fwd_split(const void *q, const void *k, const void *v, float *o, float *lse,
                 void *workspace, int nsplit, int B, int H, int N, int d, float scale, int dtype,
                 void *stream) {
  bool empty = false;
  int kps = 0, used = 0;
  int rc = split_check(q, k, v, o, lse, nsplit, B, H, N, d, scale, dtype, &empty, &kps, &used);
  if (rc != FA_OK || empty) return rc;
  if (!workspace || !aligned(workspace, 256)) return FA_ERR_WORKSPACE;
  rc = device_ready();
  if (rc != FA_OK) return rc;
  return split_launch(q, k, v, o, lse, static_cast<char *>(workspace), nsplit, B, H, N, d, scale,
                      dtype, kps, used, stream);
}

int fa_fwd_split_noalloc(const void *q, const void *k, const void *v, float *o, float *lse,
                         int nsplit, int B, int H, int N, int d, float scale, int dtype,
                         void *stream) {
  bool empty = false;
  int kps = 0, used = 0;
  int rc = split_check(q, k, v, o, lse, nsplit, B, H, N, d, scale, dtype, &empty, &kps, &used);
  if (rc != FA_OK || empty) return rc;
  if (fa_fwd_split_workspace_bytes(B, H, N, d, nsplit) > FA_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  void *ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != FA_OK) return rc;
  return split_launch(q, k, v, o, lse, static_cast<char *>(ws), nsplit, B, H, N, d, scale, dtype,
                      kps, used, stream);
}

size_t fa_naive_workspace_bytes(int B, int H, int N, int dtype) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return 0;
  if (B < 0 || H < 0 || N < 0) return 0;
  const unsigned __int128 n = (unsigned __int128)(uint64_t)B * (uint64_t)H * (uint64_t)N *
                              (uint64_t)N * (uint64_t)elem_bytes(dtype);
  const unsigned __int128 rounded = (n + 255) / 256 * 256;
  if (rounded > (unsigned __int128)std::numeric_limits<size_t>::max())
    return std::numeric_limits<size_t>::max();
  return (size_t)rounded;
}

int fa_naive_fwd(const void *q, const void *k, const void *v, float *o, float *lse, void *s_ws,
                 void *p_ws, int B, int H, int N, int d, float scale, int dtype, void *stream) {
  bool empty = false;
  int rc = check_args(q, k, v, o, lse, B, H, N, d, scale, dtype, &empty);
  if (rc != FA_OK || empty) return rc;
  if (!s_ws || !p_ws || !aligned(s_ws, 16) || !aligned(p_ws, 16)) return FA_ERR_WORKSPACE;
  if (fa_naive_workspace_bytes(B, H, N, dtype) == std::numeric_limits<size_t>::max())
    return FA_ERR_SHAPE;
  rc = device_ready();
  if (rc != FA_OK) return rc;
  return hip_status(fa::launch_naive(make_problem(q, k, v, o, lse, B, H, N, d, scale, dtype), s_ws,
                                     p_ws, static_cast<hipStream_t>(stream)));
}

// Workspace of the backward pass: dO in the input type, then lse2 and D (one float per
// row each), every part starting on a 256-byte boundary.
namespace {
struct BwdLayout {
  unsigned __int128 do16, lse2, d, total;
};
unsigned __int128 round256(unsigned __int128 n) { return (n + 255) / 256 * 256; }
BwdLayout bwd_layout(int B, int H, int N, int d, int dtype) {
  const unsigned __int128 rows = (unsigned __int128)(uint64_t)B * (uint64_t)H * (uint64_t)N;
  BwdLayout L;
  L.do16 = 0;  // fp32 inputs use dO as given: no rounded copy
  L.lse2 = dtype == FA_F32 ? 0 : round256(rows * (uint64_t)d * 2);
  L.d = L.lse2 + round256(rows * 4);
  L.total = L.d + round256(rows * 4);
  return L;
}
bool bwd_supported(int d, int dtype) {
  if (dtype == FA_F32) return d == 64 || d == 128;
  return (dtype == FA_F16 || dtype == FA_BF16) && (d == 64 || d == 128 || d == 256);
}
}  // namespace

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype) {
  if (!bwd_supported(d, dtype) || B < 0 || H < 0 || N < 0) return 0;
  const unsigned __int128 t = bwd_layout(B, H, N, d, dtype).total;
  if (t > (unsigned __int128)std::numeric_limits<size_t>::max())
    return std::numeric_limits<size_t>::max();
  return (size_t)t;
}

int fa_bwd(const void *q, const void *k, const void *v, const float *o, const float *lse,
           const float *dout, float *dq, float *dk, float *dv, void *workspace, int B, int H,
           int N, int d, float scale, int dtype, void *stream) {
  bool empty = false;
  int rc = check_args(q, k, v, o, lse, B, H, N, d, scale, dtype, &empty);
  if (rc != FA_OK) return rc;
  if (!bwd_supported(d, dtype)) return FA_ERR_HEADDIM;  // fp32 inputs at d = 256
  if (empty) return FA_OK;
  if (!dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return FA_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 256)) return FA_ERR_WORKSPACE;
  rc = device_ready();
  if (rc != FA_OK) return rc;
  const BwdLayout L = bwd_layout(B, H, N, d, dtype);
  char *ws = static_cast<char *>(workspace);
  fa::BwdProblem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.ws_do16 = ws + (size_t)L.do16;
  p.ws_lse2 = reinterpret_cast<float *>(ws + (size_t)L.lse2);
  p.ws_d = reinterpret_cast<float *>(ws + (size_t)L.d);
  p.B = B;
  p.H = H;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.dtype = dtype;
  return hip_status(fa::launch_bwd(p, static_cast<hipStream_t>(stream)));
}

// Workspace of the split backward: fa_bwd's workspace, then 3 nsplit slots of partial
// gradients (B H N d floats each), 256-byte aligned.
namespace {
unsigned __int128 bwd_split_parts_offset(int B, int H, int N, int d, int dtype) {
  return bwd_layout(B, H, N, d, dtype).total;
}
unsigned __int128 bwd_split_total(int B, int H, int N, int d, int dtype, int nsplit) {
  const unsigned __int128 slot = (unsigned __int128)(uint64_t)B * (uint64_t)H * (uint64_t)N *
                                 (uint64_t)d * 4;
  return bwd_split_parts_offset(B, H, N, d, dtype) + round256(slot * 3 * (uint64_t)nsplit);
}
}  // namespace

size_t fa_bwd_split_workspace_bytes(int B, int H, int N, int d, int dtype, int nsplit) {
  if (!bwd_supported(d, dtype) || B < 0 || H < 0 || N < 0) return 0;
  if (nsplit < 1 || nsplit > FA_MAX_SPLIT) return 0;
  const unsigned __int128 t = bwd_split_total(B, H, N, d, dtype, nsplit);
  if (t > (unsigned __int128)std::numeric_limits<size_t>::max())
    return std::numeric_limits<size_t>::max();
  return (size_t)t;
}

int fa_bwd_split_suggest(int B, int H, int N, int d, int compute_units) {
  if (B <= 0 || H <= 0 || N <= 0 || compute_units <= 0) return 1;
  if (d != 64 && d != 128 && d != 256) return 1;
  // 128 keys or queries per workgroup; the query-owned kernel holds two workgroups per
  // compute unit, so the grid is full at twice the unit count
  const int64_t wgs = int64_t(B) * H * ((N + 127) / 128);
  const int64_t full = 2 * int64_t(compute_units);
  if (wgs >= full) return 1;
  const int64_t want = (full + wgs - 1) / wgs;
  const int64_t cap = std::max<int64_t>(1, ((N + 63) / 64) / 8);  // >= 8 tiles per range
  return int(std::min<int64_t>({want, cap, int64_t(FA_MAX_SPLIT)}));
}

int fa_bwd_split(const void *q, const void *k, const void *v, const float *o, const float *lse,
                 const float *dout, float *dq, float *dk, float *dv, void *workspace, int nsplit,
                 int B, int H, int N, int d, float scale, int dtype, void *stream) {
  bool empty = false;
  int rc = check_args(q, k, v, o, lse, B, H, N, d, scale, dtype, &empty);
  if (rc != FA_OK) return rc;
  if (!bwd_supported(d, dtype)) return FA_ERR_HEADDIM;  // fp32 inputs at d = 256
  if (nsplit < 1 || nsplit > FA_MAX_SPLIT) return FA_ERR_SHAPE;
  if (empty) return FA_OK;
  if (!dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return FA_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 256)) return FA_ERR_WORKSPACE;
  const int tiles = (N + 63) / 64;
  const int tps = (tiles + nsplit - 1) / nsplit;
  const int used = (tiles + tps - 1) / tps;
  if (int64_t(B) * H * ((int64_t(N) + 127) / 128) * used > fa::kMaxGrid) return FA_ERR_SHAPE;
  rc = device_ready();
  if (rc != FA_OK) return rc;
  const BwdLayout L = bwd_layout(B, H, N, d, dtype);
  char *ws = static_cast<char *>(workspace);
  fa::BwdProblem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.ws_do16 = ws + (size_t)L.do16;
  p.ws_lse2 = reinterpret_cast<float *>(ws + (size_t)L.lse2);
  p.ws_d = reinterpret_cast<float *>(ws + (size_t)L.d);
  p.B = B;
  p.H = H;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.dtype = dtype;
  float *parts = reinterpret_cast<float *>(ws + (size_t)bwd_split_parts_offset(B, H, N, d, dtype));
  return hip_status(fa::launch_bwd_split(p, parts, used, tps, static_cast<hipStream_t>(stream)));
}

const char *fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid or too large B, H or N";
    case FA_ERR_HEADDIM: return "head dimension must be 64, 128 or 256 (fp32 backward: 64, 128)";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_WORKSPACE: return "workspace NULL or misaligned";
    case FA_ERR_HIP: return "HIP error (no device or launch failure)";
    case FA_ERR_SCRATCH: return "problem needs more than the library's static scratch";
    default: return "unknown status";
  }
}

const char *fa_version(void) { return "exact_attention_90_amd 0.1.0 gfx950"; }

int fa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
