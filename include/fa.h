/*
 * fa.h - C boundary of the gfx950 attention forward library (libfa.so).
 *
 * The library computes non-causal scaled dot-product attention
 *
 *     O = softmax(scale * Q K^T) V,      LSE = log(sum_j exp(scale * q_i . k_j))
 *
 * for every batch b, head h and query row i.  The operation is the attention
 * formula and its three-step standard form in the MUSA SDK guide
 * "FlashAttention optimization" (sections "Standard attention formula" and
 * "three-step computation"), computed the way that guide's "FlashAttention
 * complete algorithm" formula prescribes: Q blocks stay on chip while K/V blocks
 * stream past, a running row max m and row sum l are kept per query row, the
 * output accumulator is rescaled by exp(m_old - m_new) before each new P V
 * block is added, and O / l is written at the end (steps 1-4, a-f).  The
 * N x N score and probability matrices never reach device memory.
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, contiguous, row-major with the head dimension fastest:
 *       q, k, v : [B, H, N, d] of the input dtype (see fa_dtype)
 *       o       : [B, H, N, d] float32 (always float32, whatever the input dtype)
 *       lse     : [B, H, N]    float32, natural logarithm
 *   - All tensor pointers are device memory owned by the caller.  The library
 *     never allocates, frees or retains them.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     enqueue work and return; results are valid once the stream has reached
 *     the enqueued work (e.g. after hipStreamSynchronize).
 *   - Argument checks run on the host before anything is enqueued.  On any error
 *     nothing is launched and outputs are untouched.
 *   - NaN or Inf inside q, k or v is not checked; it propagates to the outputs.
 *   - All entry points are thread-safe; the library keeps no mutable state other
 *     than a per-thread copy of the last HIP error code and, per kernel, an atomic
 *     record of the devices on which its dynamic-LDS limit has been raised.
 */
#ifndef EXACT_ATTENTION_90_AMD_FA_H
#define EXACT_ATTENTION_90_AMD_FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input element type of q, k and v. */
enum fa_dtype {
    FA_F32 = 0,  /* IEEE binary32 */
    FA_F16 = 1,  /* IEEE binary16 */
    FA_BF16 = 2  /* bfloat16 (upper half of a binary32) */
};

/* Return codes.  FA_OK is 0; every error is positive. */
enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer is NULL (and the problem is not empty) */
    FA_ERR_SHAPE = 2,     /* B, H or N negative, or too large: B*H*ceil(N/128) > 2^24
                             workgroups, or one head's N*d*elem > 2^31 - 2^17 bytes */
    FA_ERR_HEADDIM = 3,   /* d is not 64, 128 or 256 (fa_bwd with FA_F32: 64 or 128) */
    FA_ERR_DTYPE = 4,     /* dtype is not one of fa_dtype */
    FA_ERR_SCALE = 5,     /* scale is not a finite number > 0 */
    FA_ERR_ALIGN = 6,     /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
    FA_ERR_WORKSPACE = 7, /* a workspace pointer is NULL or misaligned */
    FA_ERR_HIP = 8,       /* no usable HIP device, or a launch failed; see fa_last_hip_error */
    FA_ERR_SCRATCH = 9    /* fa_fwd_split_noalloc: the problem needs more than FA_SCRATCH_BYTES
                             of scratch */
};

/*
 * fa_fwd - fused attention forward (FlashAttention).
 *
 *   q, k, v  device pointers, [B, H, N, d] contiguous, element type `dtype`,
 *            16-byte aligned.
 *   o        device pointer, [B, H, N, d] float32, 16-byte aligned.  Receives
 *            O = softmax(scale * Q K^T) V.
 *   lse      device pointer, [B, H, N] float32, 4-byte aligned.  Receives
 *            m + ln(l): the natural log of sum_j exp(scale * q_i . k_j).
 *   B, H, N  batch, heads, sequence length (queries = keys = N).  Any value >= 0;
 *            N need not be a multiple of any tile size.  If B*H*N == 0 the call
 *            checks its other arguments and returns FA_OK without launching
 *            (pointers may then be NULL).
 *   d        head dimension: 64, 128 or 256 (every dtype).
 *   scale    softmax scale, finite and > 0 (usually 1/sqrt(d)).  It multiplies
 *            the float32 dot products; it is never folded into 16-bit inputs.
 *   dtype    FA_F32, FA_F16 or FA_BF16.
 *   stream   hipStream_t as void*.
 *
 * Precision: products of q and k run on the matrix cores in the input type with
 * float32 accumulation; softmax statistics are float32.  The probabilities P
 * enter the P V product as binary16 for FA_F16 and FA_BF16 inputs (for bfloat16
 * inputs V is widened exactly to binary16 on chip; |v| must stay below 65504)
 * and as float32 for FA_F32 inputs.  Results are bitwise identical from run to
 * run for the same inputs and device.
 *
 * Returns FA_OK or an fa_status error code.
 */
int fa_fwd(const void *q, const void *k, const void *v, float *o, float *lse, int B, int H, int N,
           int d, float scale, int dtype, void *stream);

/*
 * fa_fwd_stats - fa_fwd that also records the online-softmax statistics of every query
 * row after every 64-key block, for validation: the second layer of the three-layer check
 * in the CK/MI50 notes (section 4.1) compares each block's running max and running sum
 * with the standard softmax, here with the CPU oracle's blockwise recurrences (MUSA
 * guide, online-softmax recurrences m_new = max(m, max_j s_j), l_new = l e^(m - m_new) +
 * sum_j e^(s_j - m_new)).  Same kernels as fa_fwd in a statistics-recording form; O and
 * LSE are fa_fwd's.
 *
 *   q, k, v, o, lse, B, H, N, d, scale, dtype, stream   as for fa_fwd.
 *   stats   caller-owned float32 device memory of fa_fwd_stats_bytes(B, H, N) bytes,
 *           16-byte aligned (else FA_ERR_WORKSPACE): for row r = (b H + h) N + i and
 *           block t = 0 .. ceil(N/64) - 1, stats[(r ceil(N/64) + t) 2 + 0] is the kernel's
 *           running reference in base-2 units, log2(e) times the scaled score max over
 *           keys 0 .. 64 t + 63 (at d >= 128 for 16-bit inputs a lagging reference at
 *           most 8 below it, see the kernel), and stats[... + 1] the running sum of
 *           exp2(log2(e) s_j - reference) over those keys.
 * Returns FA_OK or an fa_status error code (as fa_fwd, plus FA_ERR_WORKSPACE).
 */
int fa_fwd_stats(const void *q, const void *k, const void *v, float *o, float *lse,
                 float *stats, int B, int H, int N, int d, float scale, int dtype, void *stream);

/* fa_fwd_stats_bytes - bytes of fa_fwd_stats' stats buffer: B H N ceil(N/64) 2 floats
 * (0 for negative sizes, SIZE_MAX on overflow). */
size_t fa_fwd_stats_bytes(int B, int H, int N);

/* Largest number of key ranges fa_fwd_split accepts. */
#define FA_MAX_SPLIT 64

/*
 * fa_fwd_split - fa_fwd with the keys of every head cut into ranges, for shapes
 * with few heads and long sequences (B*H*ceil(N/256) well below the number of
 * compute units), where one workgroup per Q tile leaves the device idle.
 *
 * The keys are cut into nsplit ranges of whole 64-key tiles (ceil(ceil(N/64) /
 * nsplit) tiles each; ranges that would start at or past N are dropped, so fewer
 * than nsplit may run).  For each range g the fused kernel computes every query
 * row's attention over that range alone: O_g (normalised by the range's own row
 * sum) and LSE_g.  A second kernel merges the ranges with the two-block update of
 * normalised partial outputs in the Triton tutorial (section 2.3), which is the
 * online-softmax block update of the MUSA guide (step e) applied to whole blocks:
 *     LSE = log sum_g exp(LSE_g),     O = sum_g exp(LSE_g - LSE) O_g.
 * The same rule combines the partial results of a sequence split across GPUs.
 *
 *   q, k, v, o, lse, B, H, N, d, scale, stream   as for fa_fwd.
 *   dtype      FA_F32, FA_F16 or FA_BF16.
 *   nsplit     1 .. FA_MAX_SPLIT (else FA_ERR_SHAPE).  nsplit = 1 gives results
 *              bitwise equal to fa_fwd's.
 *   workspace  caller-owned device memory of fa_fwd_split_workspace_bytes(B, H, N,
 *              d, nsplit) bytes, 256-byte aligned (else FA_ERR_WORKSPACE): the
 *              partial O_g (float32, nsplit x [B, H, N, d]) and LSE_g (float32,
 *              nsplit x [B, H, N]).  Its contents on entry do not matter; it must
 *              not be used by other work on the device until the call completes.
 *
 * Precision as for fa_fwd; the merge adds one float32 exp and multiply-add per
 * range and element.  Results are bitwise identical from run to run.
 * Returns FA_OK or an fa_status error code.
 */
int fa_fwd_split(const void *q, const void *k, const void *v, float *o, float *lse,
                 void *workspace, int nsplit, int B, int H, int N, int d, float scale, int dtype,
                 void *stream);

/* Bytes of the library's own static device scratch used by fa_fwd_split_noalloc. */
#define FA_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * fa_fwd_split_noalloc - fa_fwd_split without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code being captured into
 * a HIP graph, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The partial O_g and LSE_g go to a static device array of FA_SCRATCH_BYTES (64 MiB)
 * that the library holds on every device it runs on until the process ends.  The call
 * allocates and frees nothing (the array's device address is looked up once per device
 * on the first call there).  The kernels and results are fa_fwd_split's: bitwise equal
 * for the same arguments.
 *
 *   arguments  as for fa_fwd_split, minus workspace.
 *
 * Every call on one device shares that device's array, and a call may leave its
 * contents there: calls that can overlap on one device (several streams, several host
 * threads) race on it and must be serialised by the caller.  Nothing in the array needs
 * to start at zero (every partial the merge reads is written first).
 * Returns FA_OK, the error codes of fa_fwd_split, or FA_ERR_SCRATCH (before anything is
 * enqueued) when fa_fwd_split_workspace_bytes(B, H, N, d, nsplit) > FA_SCRATCH_BYTES.
 */
int fa_fwd_split_noalloc(const void *q, const void *k, const void *v, float *o, float *lse,
                         int nsplit, int B, int H, int N, int d, float scale, int dtype,
                         void *stream);

/*
 * fa_fwd_split_suggest - the number of key ranges for fa_fwd_split on a device with
 * `compute_units` compute units (256 on MI355X): 1 when fa_fwd's grid (one workgroup
 * per head and 256 query rows at d = 128, 128 rows otherwise) already has at least one
 * workgroup per compute unit, else enough ranges to reach that, capped so that every
 * range keeps at least 8 key tiles (512 keys) and at FA_MAX_SPLIT.  Pure arithmetic on
 * its arguments; returns 1 for empty or invalid sizes.
 */
int fa_fwd_split_suggest(int B, int H, int N, int d, int compute_units);

/*
 * Workspace bytes fa_fwd_split needs for these sizes: nsplit * B * H * N * (d + 1)
 * float32 values, each of the two parts rounded up to 256 bytes.  0 for negative
 * sizes, d not in {64, 128, 256} or nsplit outside 1 .. FA_MAX_SPLIT; SIZE_MAX if
 * the size does not fit a size_t.
 */
size_t fa_fwd_split_workspace_bytes(int B, int H, int N, int d, int nsplit);

/*
 * fa_naive_fwd - the materialised three-kernel contrast path (not for production).
 *
 * Same arguments and outputs as fa_fwd, plus two caller-owned device workspaces
 * that receive, in the input dtype, the full score matrix S = scale * Q K^T and
 * the probability matrix P = softmax(S), each [B, H, N, N] row-major
 * (the standard three steps of the MUSA guide; the Triton tutorial's section 1
 * sizes these tensors).  Three kernels run in order on `stream`: scores, row
 * softmax (which also writes lse), and O = P V.  Each kernel accumulates in
 * float32; S and P are rounded to the input dtype when stored.
 *
 *   s_ws, p_ws  device pointers of at least fa_naive_workspace_bytes(B, H, N,
 *               dtype) bytes each, 16-byte aligned, not overlapping each other
 *               or any tensor.  NULL or misaligned -> FA_ERR_WORKSPACE.
 */
int fa_naive_fwd(const void *q, const void *k, const void *v, float *o, float *lse, void *s_ws,
                 void *p_ws, int B, int H, int N, int d, float scale, int dtype, void *stream);

/*
 * Bytes of ONE naive-path workspace: B * H * N * N * sizeof(dtype), rounded up
 * to a multiple of 256.  Returns 0 for an invalid dtype or a negative size, and
 * SIZE_MAX if the product does not fit in size_t.
 */
size_t fa_naive_workspace_bytes(int B, int H, int N, int dtype);

/*
 * fa_bwd - attention backward: the gradients of O with respect to Q, K and V.
 *
 * The method is the recomputation of the pwwt.cn Triton tutorial (sections 2.4 and
 * 4.4): P is not stored; it is rebuilt tile by tile from q, k and the forward pass's
 * lse, and the chain rule gives, for the upstream gradient dO of O,
 *     dV = P^T dO,  dP = dO V^T,  D_i = <dO_i, O_i>,  dS = P * (dP - D),
 *     dQ = scale dS K,  dK = scale dS^T Q.
 * LSE is an auxiliary output and receives no gradient.
 *
 *   q, k, v    as for fa_fwd (FA_F32 inputs: d = 64 or 128).
 *   o, lse     fa_fwd's outputs for the same q, k, v and scale (device, float32).
 *   dout       device pointer, [B, H, N, d] float32, 16-byte aligned: dO.
 *   dq, dk, dv device pointers, [B, H, N, d] float32, 16-byte aligned, not overlapping
 *              any input: receive the gradients.
 *   workspace  device pointer of at least fa_bwd_workspace_bytes(B, H, N, d, dtype)
 *              bytes, 256-byte aligned, owned by the caller, not overlapping any tensor.
 *              It receives dO rounded to the input type and two floats per row.
 *   B, H, N, scale, stream as for fa_fwd.
 *
 * Precision: every product runs on the matrix cores in the input type with float32
 * accumulation; for FA_F16 and FA_BF16 inputs dO, P and dS are rounded to the input
 * type (round to nearest even) for the products that take them, for FA_F32 inputs
 * nothing is rounded below float32; D and the softmax statistics are float32.
 * Three kernels run in order on `stream` (four at d = 256, where dV and dK take one
 * launch each); results are bitwise identical from run to run (no atomics).
 *
 * Returns FA_OK, or (before any launch) the error codes of fa_fwd, FA_ERR_HEADDIM for
 * FA_F32 inputs with d = 256, FA_ERR_NULL for a NULL dout/dq/dk/dv,
 * FA_ERR_ALIGN, or FA_ERR_WORKSPACE for a NULL or misaligned workspace.
 */
int fa_bwd(const void *q, const void *k, const void *v, const float *o, const float *lse,
           const float *dout, float *dq, float *dk, float *dv, void *workspace, int B, int H,
           int N, int d, float scale, int dtype, void *stream);

/*
 * Bytes of the backward workspace: B*H*N*d*2 (dO rounded to a 16-bit input type; none
 * for FA_F32) + 8*B*H*N, each of its parts rounded up to a multiple of 256.  Returns 0 for a combination fa_bwd does not
 * support or a negative size, and SIZE_MAX if the total does not fit in size_t.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype);

/*
 * fa_bwd_split - fa_bwd for few heads and long sequences.  dK and dV are sums over
 * query rows, and dQ a sum over key rows, of per-pair terms (the chain rule through
 * O = P V and the softmax, as in fa_bwd).  Here the key-owned kernel's query tiles and
 * the query-owned kernel's key tiles (64 rows each) are cut into up to nsplit ranges of
 * ceil(ceil(N/64) / nsplit) tiles; every range writes its partial dQ, dK and dV to its
 * own slot of the workspace, and a last kernel adds the slots in range order into dq,
 * dk and dv.  Results are bitwise identical from run to run; nsplit = 1 gives fa_bwd's.
 *
 *   all arguments but workspace and nsplit   as for fa_bwd.
 *   dtype      as for fa_bwd (FA_F32: d = 64 or 128).
 *   nsplit     1 .. FA_MAX_SPLIT (else FA_ERR_SHAPE).
 *   workspace  fa_bwd_split_workspace_bytes(B, H, N, d, dtype, nsplit) bytes of device
 *              memory, 256-byte aligned: fa_bwd's workspace followed by 3 nsplit
 *              float32 slots of [B, H, N, d].
 *
 * Returns FA_OK or an fa_status error code.
 */
int fa_bwd_split(const void *q, const void *k, const void *v, const float *o, const float *lse,
                 const float *dout, float *dq, float *dk, float *dv, void *workspace, int nsplit,
                 int B, int H, int N, int d, float scale, int dtype, void *stream);

/* Workspace bytes of fa_bwd_split: fa_bwd_workspace_bytes(B, H, N, d, dtype) plus
 * 3 * nsplit * B * H * N * d float32 values rounded up to 256 bytes.  0 for an
 * unsupported dtype or d, negative sizes or nsplit outside 1 .. FA_MAX_SPLIT; SIZE_MAX if the
 * size does not fit a size_t. */
size_t fa_bwd_split_workspace_bytes(int B, int H, int N, int d, int dtype, int nsplit);

/* fa_bwd_split_suggest - as fa_fwd_split_suggest, for the backward pass's grids (one
 * workgroup per head and 128 keys or queries; the query-owned kernel holds two per
 * compute unit): the number of ranges that gives the grids two workgroups per compute
 * unit, each range keeping at least 8 tiles; 1 when the grid is already that large or
 * the sizes are empty or invalid. */
int fa_bwd_split_suggest(int B, int H, int N, int d, int compute_units);

/* Static, human-readable text for a status code (never NULL). */
const char *fa_status_string(int status);

/* Static version string of the library, e.g. "exact_attention_90_amd 0.1.0 gfx950". */
const char *fa_version(void);

/* The hipError_t value behind the calling thread's most recent FA_ERR_HIP (0 if none). */
int fa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_90_AMD_FA_H */
