/*
 * msa.h - C ABI of the MI355X (gfx950) MiniMax Sparse Attention training hot path.
 *
 * What is computed (sources are the three pages on Flash-MSA / MiniMax Sparse
 * Attention; the method is described in prose only):
 *
 *   Index Branch  - msa_proxy_select
 *     One proxy head per GQA group scores each query against every causal key,
 *     the scores are max-pooled over 128-key blocks, and the top-k blocks of
 *     each query are kept as that query's block-index cache.
 *     ("Flash-MSA: Open-Source Sparse Attention Kernels Debut", section "How MSA
 *     works": 128-key blocks picked by max-pooling proxy scores, indices cached
 *     so only the proxy pass stays quadratic, group-wise proxy heads;
 *     ai-beat "flash-msa-sparse-attention-training", paragraphs 1, 3 and 4.)
 *
 *   Main Branch   - msa_fwd, msa_bwd
 *     Exact softmax GQA attention over only the keys of the cached blocks, and
 *     its gradients dQ, dK, dV.  (ai-beat page, paragraph 1: exact softmax over
 *     the selected blocks; paragraph 2: a backward pass through the learned
 *     sparse pattern; xcelit page, "How MSA works": GQA main attention.)
 *
 * Readings where the pages are silent (also listed with the design notes):
 *   - proxy score = plain dot product q_p . k_p (no scale, no activation);
 *   - query head h belongs to KV/proxy group g = h / (H / G);
 *   - query t may pick blocks 0 .. t/128; inside a block only keys j <= t count,
 *     for pooling and for attention; the diagonal block is an ordinary candidate;
 *   - equal pooled scores rank the lower block index first; -0 equals +0;
 *   - a cache row lists its min(topk, t/128 + 1) blocks in ascending order and
 *     is padded with -1;
 *   - softmax scale = dims.scale, or 1/sqrt(d) when dims.scale <= 0;
 *   - lse is the natural-log log-sum-exp of the scaled scores.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are device pointers owned by the caller, row-major,
 *     contiguous, 16-byte aligned.  bf16 values are passed as raw 16-bit words.
 *       qp, kp            [B, T, G, dp]  bf16
 *       q, o, dout, dq    [B, T, H, d]   bf16
 *       k, v, dk, dv      [B, T, G, d]   bf16
 *       idx               [B, G, T, topk] int32 (the block-index cache)
 *       lse               [B, T, H]      fp32
 *   - ws / ws_bytes is caller-owned device scratch memory.  msa_workspace_bytes
 *     gives the size that lets a call run in one pass over the tokens; any size
 *     at or above msa_workspace_min_bytes works (smaller sizes make the call
 *     walk the tokens in more windows).  Its contents need no initialisation
 *     and are undefined afterwards.  The library allocates no device memory.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).  All
 *     work is enqueued asynchronously on it; outputs are valid once the stream
 *     reaches that point.  Calls on one workspace must not overlap.
 *   - Argument checks happen on the host before anything is enqueued; a
 *     failing check returns an error code and enqueues nothing.  A launch
 *     failure returns MSA_ERR_HIP.  Outputs are fully overwritten.
 *   - Cache check: when the environment variable MSA_VALIDATE is set to a
 *     non-empty value other than "0" (read at every call), msa_fwd, msa_bwd
 *     and msa_fwd_bwd first check idx on the device: every entry must be -1
 *     or a causal block 0..t/128, no block may appear twice in a row, and
 *     every row must list at least one block.  The call then waits for the
 *     stream (the check's result is read back to the host) and returns
 *     MSA_ERR_INDEX without launching anything else if a row fails; the first
 *     16 bytes of ws are used for the result.  Off by default: unchecked calls
 *     never synchronise.
 *   - Supported shapes: B >= 1; T >= 128 with T % 128 == 0; H % G == 0 with
 *     R = H / G in {1, 2, 4, 8, 16}; d in {64, 128}; dp in {32, 64, 128};
 *     1 <= topk <= 1024 (topk may exceed the number of causal blocks);
 *     T * topk < 2^31; B * T < 2^30; B * G <= 65535; scale finite.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t msa_bf16; /* raw bfloat16 bits */

typedef enum {
  MSA_OK = 0,
  MSA_ERR_NULL = 1,        /* a required pointer is NULL */
  MSA_ERR_SHAPE = 2,       /* dims out of the supported range */
  MSA_ERR_UNSUPPORTED = 3, /* a head dim / proxy dim / group ratio not built */
  MSA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  MSA_ERR_WORKSPACE = 5,   /* ws_bytes below msa_workspace_min_bytes */
  MSA_ERR_HIP = 6,         /* the HIP runtime reported an error */
  MSA_ERR_INDEX = 7,       /* MSA_VALIDATE set: idx is not a valid cache (nothing else ran) */
  MSA_ERR_SCRATCH = 8      /* msa_decode_fwd_static: the problem needs more than MSA_STATIC_SCRATCH_BYTES */
} msa_status;

typedef struct {
  int32_t B, T, H, G, d, dp, topk;
  float scale; /* softmax scale; <= 0 selects 1/sqrt(d) */
} msa_dims;

typedef enum {
  MSA_OP_SELECT = 0,
  MSA_OP_FWD = 1,
  MSA_OP_BWD = 2,
  MSA_OP_DECODE_SELECT = 3, /* msa_decode_select: B*G*(T/128) fp32 pooled scores */
  MSA_OP_DECODE_FWD = 4,    /* msa_decode_fwd: B*G*topk fp32 partials of R*(d+1) values */
  MSA_OP_FWD_BWD = 5        /* msa_fwd_bwd */
} msa_op;

/* Workspace that lets `op` run at its preferred token window: all tokens for
 * MSA_OP_SELECT and MSA_OP_BWD; for MSA_OP_FWD and MSA_OP_FWD_BWD, windows
 * whose query rows of one KV group span at most 64 MiB (32768 tokens at
 * R = 8, d = 128), which keeps the forward's re-reads of those rows in the
 * last-level cache.  Capped at 80 GiB (8 GiB for MSA_OP_SELECT) for the
 * largest shapes, which are then walked in smaller windows.  Returns 0 for
 * invalid dims. */
size_t msa_workspace_bytes(const msa_dims* dims, msa_op op);

/* Smallest workspace `op` accepts (one 128-token window).  0 for invalid dims. */
size_t msa_workspace_min_bytes(const msa_dims* dims, msa_op op);

/* Index Branch.  For every (b, g, t): pooled_i = max over keys j of block i
 * with j <= t of dot(qp[b,t,g,:], kp[b,j,g,:]) (fp32), for i <= t/128; the
 * min(topk, t/128+1) highest pooled blocks (ties: lower index) are written
 * ascending to idx[b,g,t,:], the rest of the row is -1.  Reads qp and kp;
 * writes idx. */
msa_status msa_proxy_select(const msa_dims* dims, const msa_bf16* qp, const msa_bf16* kp,
                            int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* Fixed block pattern (keelcrux "Flash-MSA: Train on a million tokens without
 * breaking the compute bank", section "Under the hood": the block pattern is
 * configurable by window size and dilation; the pages define neither, this is
 * the reading).  For every (b, g, t), with nc = t/128 + 1 causal blocks, the
 * row idx_out[b,g,t,:] lists once each, in ascending order:
 *   - the `window` most recent causal blocks, max(0, nc - window) .. nc - 1;
 *   - each causal block below the window whose index is a multiple of
 *     `dilation` (none when dilation == 0);
 *   - when idx_in != NULL, each entry of idx_in[b,g,t,0..k_in) that is a
 *     causal block (other entries, -1 included, are ignored), so a proxy top-k
 *     cache can be united with the pattern;
 * and the row is padded with -1 to width dims->topk.  Only B, T, G and topk of
 * dims are read.  Requirements (MSA_ERR_SHAPE otherwise): window >= 0,
 * dilation >= 0, at least one of window, dilation, idx_in selects blocks
 * (window > 0 or dilation > 0 or idx_in != NULL, so that msa_fwd gets a valid
 * cache when idx_in rows are valid), 1 <= k_in <= 1024 when idx_in is given,
 * and dims->topk >= min(N, min(window, N) + ceil(max(0, N - window) / dilation)
 * + k_in) with N = T/128 (the largest row the pattern can produce).  No
 * workspace; idx_in and idx_out must not overlap. */
msa_status msa_pattern_select(const msa_dims* dims, int32_t window, int32_t dilation, const int32_t* idx_in,
                              int32_t k_in, int32_t* idx_out, void* stream);

/* Main Branch forward.  For every (b, t, h), g = h / (H/G), over the key set
 * J = { j <= t : j/128 is listed in idx[b,g,t,:] } and s_j = scale * q.k_j:
 *   o[b,t,h,:] = sum_j softmax(s)_j v[b,j,g,:]   (bf16, round to nearest even)
 *   lse[b,t,h] = max_j s_j + ln sum_j exp(s_j - max_j s_j)            (fp32)
 * idx must be a valid cache (entries in 0..t/128 or -1, no repeats, at least
 * one entry per row): rows produced by msa_proxy_select always are. */
msa_status msa_fwd(const msa_dims* dims, const msa_bf16* q, const msa_bf16* k, const msa_bf16* v,
                   const int32_t* idx, msa_bf16* o, float* lse, void* ws, size_t ws_bytes,
                   void* stream);

/* Main Branch backward of L = sum(o * dout) through the same sparse pattern,
 * with P_j = exp(s_j - lse), D = dot(dout, o) (o as stored in bf16),
 * dS_j = P_j (dot(dout, v_j) - D):
 *   dq[b,t,h,:] = scale * sum_j dS_j k_j
 *   dk[b,j,g,:] = scale * sum_{t,h in g} dS_{t,h,j} q[b,t,h,:]
 *   dv[b,j,g,:] =         sum_{t,h in g} P_{t,h,j} dout[b,t,h,:]
 * (keys no query reads get zero gradients).  o and lse are msa_fwd's outputs
 * for the same q, k, v, idx.  No gradient flows to qp/kp: the top-k choice is
 * piecewise constant. */
msa_status msa_bwd(const msa_dims* dims, const msa_bf16* q, const msa_bf16* k, const msa_bf16* v,
                   const msa_bf16* o, const msa_bf16* dout, const float* lse, const int32_t* idx,
                   msa_bf16* dq, msa_bf16* dk, msa_bf16* dv, void* ws, size_t ws_bytes,
                   void* stream);

/* Merged forward and backward (keelcrux "Flash-MSA: Train on a million tokens
 * without breaking the compute bank", section "The fact": forward and backward
 * kernels are merged; section "Under the hood": activation memory cut about
 * fivefold; the pages give no mechanism, this is the reading).  For a training
 * step that runs a layer's backward right after its forward (the recompute
 * pattern: between the two only q, k, v and the block-index cache are kept,
 * not o and lse), one call writes o, lse exactly as msa_fwd and dq, dk, dv as
 * msa_bwd given that o:
 *   - each token window builds one inverse index that both halves use;
 *   - D = rowsum(dout * o) of the bf16 o is formed by the forward combine
 *     while o is in registers (no separate pass over o and dout);
 *   - the dQ partials reuse the forward partials' workspace.
 * Same layouts, shape rules and errors as msa_fwd / msa_bwd; dout is read,
 * o and lse are written. */
msa_status msa_fwd_bwd(const msa_dims* dims, const msa_bf16* q, const msa_bf16* k, const msa_bf16* v,
                       const msa_bf16* dout, const int32_t* idx, msa_bf16* o, float* lse, msa_bf16* dq, msa_bf16* dk,
                       msa_bf16* dv, void* ws, size_t ws_bytes, void* stream);

/* ---- Decode step: one new query per sequence against its caches.
 * ai-beat "flash-msa-sparse-attention-training", paragraph 1: MSA also serves
 * inference (prefill and decode).  Prefill is msa_proxy_select + msa_fwd on
 * the prompt.  A decode step computes for the new token of each sequence what
 * those two compute for its row: with t = len[b] - 1 the new token's position,
 * its own key, value and proxy key already written at position t of the caches.
 *
 * Layouts (device pointers, contiguous, 16-byte aligned):
 *   qp  [B, G, dp]  bf16    proxy query of the new token
 *   q   [B, H, d]   bf16    query heads of the new token; o the same shape
 *   kp  [B, T, G, dp], k, v [B, T, G, d]  bf16 caches of capacity T tokens
 *   len [B]         int32   tokens cached per sequence, the new one included
 *   idx [B, G, topk] int32  block-index row of the new token
 *   lse [B, H]      fp32
 * dims: B, T (cache capacity; T % 128 == 0), H, G, d, dp, topk and scale as
 * for the training entry points (msa_decode_select reads B, T, G, dp, topk).
 * len values are read on the device: a sequence whose len is outside 1..T gets
 * an all -1 idx row, o = 0 and lse = -inf.  Cache rows at or past len are never
 * read.  ws must hold msa_workspace_bytes(dims, MSA_OP_DECODE_SELECT or
 * MSA_OP_DECODE_FWD) bytes (the minimum is the same). */

/* For every (b, g): pooled_i = max over cached keys j <= t of block i of
 * dot(qp[b,g,:], kp[b,j,g,:]) (fp32), i <= t/128; the min(topk, t/128 + 1)
 * highest blocks (ties: lower index) ascending in idx[b,g,:], -1 after. */
msa_status msa_decode_select(const msa_dims* dims, const msa_bf16* qp, const msa_bf16* kp, const int32_t* len,
                             int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* For every (b, h), g = h / (H/G), over J = { j <= t : j/128 listed in
 * idx[b,g,:] } and s_j = scale * q[b,h,:].k[b,j,g,:]:
 *   o[b,h,:] = sum_j softmax(s)_j v[b,j,g,:] (bf16),  lse[b,h] = ln sum_j exp(s_j).
 * idx entries that are -1 or above t/128 are ignored; a row with no other
 * entry gives o = 0, lse = -inf.  Blocks listed twice are counted twice, so
 * rows should be as msa_decode_select writes them. */
msa_status msa_decode_fwd(const msa_dims* dims, const msa_bf16* q, const msa_bf16* k, const msa_bf16* v,
                          const int32_t* len, const int32_t* idx, msa_bf16* o, float* lse, void* ws,
                          size_t ws_bytes, void* stream);

/* ---- Decode attention without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).
 *
 * Same arguments, layouts, results and errors as msa_decode_fwd, minus ws and
 * ws_bytes: the per-slot partials live in a static device array of
 * MSA_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The call allocates nothing.  It returns
 * MSA_ERR_SCRATCH, with nothing enqueued, when the problem needs more than
 * that, i.e. when msa_workspace_bytes(dims, MSA_OP_DECODE_FWD) exceeds
 * MSA_STATIC_SCRATCH_BYTES (16 sequences x 4 groups x top-32 x 8 heads x
 * d 128 need 8.1 MiB).  It runs on the current device, and stream must belong
 * to it (MSA_ERR_UNSUPPORTED otherwise).  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  No part of the array needs
 * to start at zero: each call writes every partial it reads. */
#define MSA_STATIC_SCRATCH_BYTES (16u << 20)
msa_status msa_decode_fwd_static(const msa_dims* dims, const msa_bf16* q, const msa_bf16* k, const msa_bf16* v,
                                 const int32_t* len, const int32_t* idx, msa_bf16* o, float* lse, void* stream);

/* ---- Optional launch timing, for benchmarks and profiling tools.
 * When enabled, the library records a pair of HIP events on the call's stream
 * around every launch of the kernels listed below (the inverse-index build
 * counts as one launch of four kernels).  Timing state belongs to the calling
 * host thread: msa_timing_enable and msa_timing_read act on the launches that
 * thread made, and threads never share it.  It is off by default and costs
 * nothing when off.  At most 4096 launches are recorded between two
 * msa_timing_enable calls; later launches run untimed.  A thread's events are
 * created on first use and kept until the process ends. */
typedef enum {
  MSA_K_PROXY_POOL = 0,   /* proxy score + block max-pool */
  MSA_K_TOPK = 1,         /* per-row top-k -> idx */
  MSA_K_INVERSE = 2,      /* block -> pair inverse index (4 kernels) */
  MSA_K_FWD_PARTIALS = 3, /* forward per-pair partials (KV-stationary) */
  MSA_K_FWD_COMBINE = 4,  /* forward log-sum-exp combine */
  MSA_K_BWD_DOT = 5,      /* D = rowsum(dout * o) and accumulator clears */
  MSA_K_BWD_PARTIALS = 6, /* backward dK/dV + per-pair dQ partials (KV-stationary) */
  MSA_K_DQ_COMBINE = 7,   /* dQ partial sums */
  MSA_K_CONVERT = 8,      /* fp32 -> bf16 of dK, dV */
  MSA_K_PATTERN = 9,      /* fixed window/dilation pattern (msa_pattern_select) */
  MSA_K_DEC_POOL = 10,    /* decode: proxy scores of the new query + block max-pool */
  MSA_K_DEC_TOPK = 11,    /* decode: top-k of each (sequence, group) row */
  MSA_K_DEC_ATTN = 12,    /* decode: per-slot attention partials */
  MSA_K_DEC_COMBINE = 13, /* decode: log-sum-exp merge of the slots */
  MSA_K_COUNT = 14
} msa_kernel_id;

/* on != 0 enables timing; any call clears what was recorded. */
void msa_timing_enable(int on);

/* Waits for the recorded events and writes, for each msa_kernel_id k < n,
 * the summed duration in milliseconds to ms[k] and the number of timed
 * launches to launches[k] (either array may be NULL).  Returns MSA_OK, or
 * MSA_ERR_HIP if an event could not be read. */
msa_status msa_timing_read(double* ms, int32_t* launches, int32_t n);

/* Static description of a status code (never NULL). */
const char* msa_status_str(msa_status s);

/* Library version string, e.g. "msa-gfx950 0.1". */
const char* msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
