/*
 * attn_softcap.h -- C ABI of a fused attention forward and backward for the
 * AMD MI355X (gfx950) with tanh logit soft-capping and a softmax sink.
 *
 * What is computed (per batch row b, query head h, query i, key j; the KV
 * head of h is h / (Hq/Hkv), so GQA/MQA read K and V without copies):
 *
 *   u_ij  = scale * <q_i, k_j> + bias_ij                  (bias optional)
 *   s_ij  = softcap * tanh(u_ij / softcap)   if softcap > 0, else s_ij = u_ij
 *   visible(i,j) = same packed segment  and  (!causal or j <= i)  and
 *                  (window <= 0 or (causal ? i-j < window : |i-j| < window))
 *   softmax over the visible j of row i, plus one sink column of logit
 *   sigma_h counted exactly once per row (sink modes below);
 *   out_i = sum_j P_ij v_j,   lse_i = ln(sum_j e^{s_ij} + [sink] e^{sigma_h}).
 *
 * Sources (cited by page title and section):
 *  - "Thread tanh logit softcapping through FlashAttention (FA2, opt-in
 *    FA3)", intro and "What changed": the cap cap*tanh(x/cap) on attention
 *    logits; softcap = 0 is the default and changes nothing; a requested cap
 *    is never dropped silently (every entry point fails closed instead).
 *  - "Support logits soft-capping in the Pallas-Triton attention VJP", PR
 *    description: the cap goes after the bias add and before masking; the
 *    backward chains 1 - tanh(u/c)^2 into ds, taken before masking, and dk
 *    and dbias are gradients with respect to the pre-cap logits.
 *  - MaxText commit message quoted on that page: packed segments (causal
 *    inside each segment), varlen cu_seqlens, sliding window, native GQA,
 *    head_dim above 256.
 *  - "learnable softmax sink with context-parallel p2p" (TransformerEngine
 *    PR #3551), "What changed": softmax_type learnable / off-by-one, one
 *    offset per head, the sink as one more softmax column counted once per
 *    query row, and its gradient summed over the query rows.
 *
 * Layouts (all contiguous, row-major):
 *  - q, out, dout, dq : [B, Sq, Hq, D]   (BSHD; SBHD [Sq, B, Hq, D]: attn_layout)
 *  - k, v, dk, dv     : [B, Sk, Hkv, D]  (SBHD [Sk, B, Hkv, D])
 *  - THD (varlen): pass cu_seqlens, B = 1 and Sq = Sk = total tokens T; the
 *    tensors are then [T, H, D], which is the same memory as [1, T, H, D].
 *  - bias, dbias      : [B, Hq, Sq, Sk], same dtype as q (or broadcast: see
 *                       attn_bias_bcast).
 *  - lse              : [B, Hq, Sq] float32, natural log, sink included.
 *  - segment_ids      : [B, Sq] int32, non-decreasing along each row (packed
 *                       rows); a key is visible only inside its own run of
 *                       equal adjacent ids (for non-decreasing ids: equal id).
 *  - cu_seqlens       : [nseq + 1] int32, cu[0] = 0, non-decreasing, cu[nseq] = T
 *                       (tokens outside [cu[0], cu[nseq]) form one run each side).
 *  - sink / dsink     : [Hq] float32.
 *
 * Ownership: the caller allocates every buffer (device memory unless noted)
 * and keeps it alive until the work on `stream` has finished.  The library
 * allocates nothing and keeps no state between calls.  `stream` is a
 * hipStream_t (NULL = the default stream); calls enqueue work and return
 * without synchronising.
 *
 * Errors: every entry point validates its arguments on the host first.  Any
 * status other than ATTN_OK means that no work was enqueued; the reason is
 * available from attn_last_error() (thread-local, valid until the next call
 * on the same thread).
 */
#ifndef ATTN_SOFTCAP_H
#define ATTN_SOFTCAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_INVALID_ARGUMENT = 1, /* a null pointer, bad size or inconsistent option */
  ATTN_UNSUPPORTED = 2,      /* a well-formed request this library does not implement */
  ATTN_HIP_ERROR = 3         /* a launch failed; nothing further was enqueued */
} attn_status;

/* Element type of q, k, v, bias, out, dout, dq, dk, dv, dbias.  bf16 and fp16
 * contract on the matrix cores with fp32 accumulation; fp32 on the fp32
 * matrix instructions.  (fp16 is listed as not covered on the learnable-sink
 * page, "Not covered"; here it takes the same kernels as bf16, built a
 * second time for fp16 elements, except that the forward keeps a running
 * maximum: probabilities relative to a fixed reference at the cap could
 * leave fp16's exponent range.  A sink that takes all but a tiny share of a
 * row's mass still leaves that row's output, and the probabilities behind
 * it, small: values below fp16's normal range (2^-14) carry an absolute
 * spacing of 2^-24 rather than 11 bits of relative precision.) */
typedef enum attn_dtype { ATTN_BF16 = 0, ATTN_FP32 = 1, ATTN_FP16 = 2 } attn_dtype;

/* Softmax sink ("softmax_type" on the learnable-sink page, "What changed"):
 * none (vanilla), off-by-one (a sink column with its logit fixed at 0 and no
 * gradient), learnable (logit sink[h], with gradient dsink[h]). */
typedef enum attn_sink_mode {
  ATTN_SINK_NONE = 0,
  ATTN_SINK_OFF_BY_ONE = 1,
  ATTN_SINK_LEARNABLE = 2
} attn_sink_mode;

/* Memory layout of q, k, v, out, out_lo, dout, dq, dk, dv (heads and the
 * head dimension contiguous in both): BSHD [B, S, H, D] or SBHD [S, B, H, D]
 * (the bshd and sbhd formats of the learnable-sink page's "Verification"
 * table).  THD (cu_seqlens) is BSHD with B = 1. */
typedef enum attn_layout { ATTN_LAYOUT_BSHD = 0, ATTN_LAYOUT_SBHD = 1 } attn_layout;

/* A bias broadcast over batch rows and/or query heads: its shape is
 * [1 or B, 1 or Hq, Sq, Sk] and dbias has the same shape, the full gradient
 * summed over the broadcast dimensions (the learnable-sink page's review
 * "Offset Corrupts Bias Gradient Shape": dbias follows the bias shape). */
typedef enum attn_bias_bcast {
  ATTN_BIAS_BCAST_BATCH = 1,
  ATTN_BIAS_BCAST_HEADS = 2
} attn_bias_bcast;

/* How the backward forms dq (the same result either way, to rounding).
 *  - ATTN_DQ_DU_BLOCKS: the dk/dv kernel hands dU = dS * (1 - tanh^2) to the
 *    dq kernel through the workspace as blocks of 32 keys x 32 queries in
 *    the element type, B*Hq*ceil(Sk/32)*ceil(Sq/32) blocks of 2 KiB (bf16,
 *    fp16) or 4 KiB (fp32): 4 GiB at B=4, Hq=32, S=4096 in bf16; only the
 *    visible blocks are written and read.  fp32 at any D; bf16 or fp16 with
 *    D = 64, 128, 256 or 512 (with a bias also Sk % 8 == 0); ATTN_UNSUPPORTED
 *    otherwise.
 *  - ATTN_DQ_RECOMPUTE: the dq kernel recomputes the logits, probabilities
 *    and dP itself; the workspace stays O(B*Hq*Sq).
 *  - ATTN_DQ_AUTO (0): DU_BLOCKS where supported, D >= 128 (or dropout is
 *    on) and its buffer is at most 16 GiB, else RECOMPUTE (at D = 64
 *    recomputing is faster without dropout).
 * The [b, h, q, kv] materialisation and its memory cost are what the MaxText
 * commit quoted on "Support logits soft-capping in the Pallas-Triton
 * attention VJP" weighs (12.5 against 3.3 GiB at 8k tokens); the blocks here
 * are in the element type and touched only where visible. */
typedef enum attn_dq_mode {
  ATTN_DQ_AUTO = 0,
  ATTN_DQ_DU_BLOCKS = 1,
  ATTN_DQ_RECOMPUTE = 2
} attn_dq_mode;

/* The problem description shared by every entry point.
 * Every tensor pointer (q, k, v, bias, out, out_lo, dout, dq, dk, dv, dbias)
 * must be 16-byte aligned: the kernels move rows 16 bytes at a time.  A
 * misaligned pointer is rejected with ATTN_INVALID_ARGUMENT before anything is
 * launched.  A zero-initialised struct plus the sizes and q/k/v is a valid
 * plain attention problem (no cap, no sink, no mask, scale 1/sqrt(D)). */
typedef struct attn_args {
  int dtype;                   /* attn_dtype of q, k, v, bias, out, dout, dq, dk, dv, dbias */
  int B, Sq, Sk, Hq, Hkv, D;   /* D in {64, 128, 256, 512}; Hq % Hkv == 0 (MaxText commit: native GQA/MQA;
                                  head_dim above 256) */
  const void* q;
  const void* k;
  const void* v;
  const void* bias;            /* nullable: additive bias after the scale, before the cap (tokamax PR
                                  description; post_scale_bias in the learnable-sink page's review) */
  const int32_t* segment_ids;  /* nullable: packed rows (needs Sq == Sk; MaxText commit: packing) */
  const int32_t* cu_seqlens;   /* nullable: THD varlen (needs B == 1, Sq == Sk); not with segment_ids */
  int nseq;                    /* number of sequences in cu_seqlens */
  int causal;                  /* nonzero: key j visible only for j <= i (needs Sq == Sk) */
  int window;                  /* <= 0: none; else causal: 0 <= i-j < window, non-causal: |i-j| < window
                                  (MaxText commit: sliding window) */
  float softcap;               /* 0: off; > 0: s = softcap * tanh(u / softcap) (TE softcap page, intro and
                                  "What changed": the softcap kwarg, 0 = off) */
  float scale;                 /* 0: 1/sqrt(D) */
  int sink_mode;               /* attn_sink_mode */
  const float* sink;           /* [Hq] sink logits; required iff sink_mode == ATTN_SINK_LEARNABLE */
  int dq_mode;                 /* attn_dq_mode (backward only; the forward ignores it) */
  /* The other two packed forms of "Support logits soft-capping in the
   * Pallas-Triton attention VJP" (PR description: k_start and a dense boolean
   * mask, agreeing to every digit with segment ids); each only removes pairs,
   * on top of causal, window and segments. */
  const int32_t* k_start;      /* nullable: [B, Sq] int32 (THD: [T]), the first key query i may see (keys
                                  j >= k_start[i]); non-decreasing along a row (the library uses its running
                                  maximum, which equals it then) */
  const uint8_t* mask;         /* nullable: [B, Sq, Sk] bytes (THD: [T, T]), nonzero = visible; 16-byte
                                  aligned.  Every tile then takes the per-pair masked path (slower) */
  int bias_bcast;              /* 0: bias and dbias are [B, Hq, Sq, Sk]; else attn_bias_bcast flags */
  int layout;                  /* attn_layout of the q- and k-side tensors (0: BSHD) */
  /* Dropout on the attention probabilities inside the kernels (the pages
   * exclude it or reject it with packing: tokamax PR description, MaxText
   * commit; the learnable-sink page's "What changed" carries the rng state
   * among the forward's outputs).  After the softmax each probability is kept
   * with probability 1 - p' and scaled by 1 / (1 - p'), where p' = floor(p *
   * 2^16) / 2^16 is p rounded down to a multiple of 2^-16 (the decisions
   * compare 16-bit draws); lse is that of the undropped softmax.  Pair (query
   * i, key j) of batch row b, query head h is kept iff 16-bit half j % 8 of
   * Philox4x32-10 at counter (j / 8, i, b * Hq + h, offset % 2^32) under key
   * (seed % 2^32, seed / 2^32) is at least floor(p * 2^16); half m is the low
   * (m even) or high (m odd) 16 bits of output word m / 2.  The backward must
   * get the same p, seed and offset.
   * bf16 / fp16 run it on the fast kernels where those take the problem (D
   * = 64 .. 256, and 512 without a bias; dq from the dU blocks, or on the
   * generic kernel with ATTN_DQ_RECOMPUTE); fp32 and the rest run the
   * generic (slower) kernels. */
  float dropout_p;             /* 0: off; in [0, 1) */
  uint64_t dropout_seed;
  uint64_t dropout_offset;
} attn_args;

/* Host-only check of `a` (no device access, nothing launched).  Returns the
 * status that attn_fwd and attn_bwd would return for `a` before looking at
 * their own pointer arguments (output pointers, workspace).  Fail closed as
 * on "Thread tanh logit softcapping through FlashAttention", "What changed":
 * a requested cap, sink or mask is never dropped; an unsupported combination
 * is ATTN_UNSUPPORTED, never a silent fallback. */
attn_status attn_validate(const attn_args* a);

/* Device workspace (bytes) that attn_fwd / attn_bwd need for `a` (0 if
 * none); (size_t)-1 if `a` is invalid.  The size depends only on `a`:
 *  - forward: two int32 [B*Sq] arrays of segment runs, only with
 *    segment_ids or cu_seqlens; with k_start one int32 [B*Sq] and one int32
 *    [B*Sk] array of visibility bounds; with a dense mask five int32 [B*Sq]
 *    and two int32 [B*Sk] arrays and one int32 per batch row (the key range
 *    of each query prepared from the mask, the query range of each key, and
 *    whether those ranges describe the mask exactly);
 *  - backward: the same, delta [B*Hq*Sq] fp32, sink-gradient partials with
 *    a learnable sink, the dU blocks when dq_mode resolves to
 *    ATTN_DQ_DU_BLOCKS (see attn_dq_mode), with a broadcast bias and dbias a
 *    full [B, Hq, Sq, Sk] dbias in the input dtype (for a bias broadcast over
 *    heads on the 16-bit D = 128 / 256 kernels, [B, Hkv*s, Sq, Sk] slabs
 *    already summed over each workgroup's heads, of which only the query
 *    rows that see some key of a key block are written and read; reduced
 *    into the caller's dbias), and for bf16 / fp16 with D = 64, 128 or 256 when
 *    B*Hkv*ceil(Sk/128) < 1024 (D = 512, with a bias only when Sk % 8 == 0:
 *    B*Hkv*ceil(Sk/32) < 1024), 2*s*B*Sk*Hkv*D*4 bytes of fp32 partial
 *    dK/dV: the dk/dv kernel then splits each GQA group's query heads over s
 *    workgroups (s the smallest divisor of Hq/Hkv reaching 1024 workgroups,
 *    else the largest), summed afterwards in a fixed order. */
size_t attn_fwd_workspace_size(const attn_args* a);
size_t attn_bwd_workspace_size(const attn_args* a);

/* Forward (tokamax PR description: cap after the bias add, before masking;
 * learnable-sink page, "What changed": the sink column counted once per row,
 * and the softmax statistics returned with the output).
 * Writes out [B,Sq,Hq,D] (dtype) and lse [B,Hq,Sq] (float32, natural log,
 * sink included).  A query row that sees no key and has no sink gets
 * out = 0, lse = -inf; with a sink, out = 0 and lse = sigma.
 * out_lo: nullable, bf16 or fp16 only, [B,Sq,Hq,D] in that type: receives the
 * part of the fp32 output that its rounding to `out` drops, out_lo = O - out
 * rounded to the type.
 * Passed on to the backward it makes delta = <dO, O> (and so dsink, which
 * sums p_sink * delta over the query rows) exact to about 16 bits instead of
 * inheriting out's 8 (bf16) or 11 (fp16); NULL keeps `out` alone.  Must be NULL
 * for fp32.
 * workspace: device buffer of at least attn_fwd_workspace_size(a) bytes,
 * 256-byte aligned (may be NULL when that size is 0); its contents on entry
 * do not matter. */
attn_status attn_fwd(const attn_args* a, void* out, float* lse, void* out_lo, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Backward by recomputation, from the forward's out, out_lo and lse and
 * dout (tokamax PR description: 1 - tanh(u/c)^2 chained into ds, taken before
 * masking; dk and dbias are gradients with respect to the pre-cap logits;
 * learnable-sink page, "What changed": the sink gradient is a sum over the
 * query rows, -sum_i p_sink(i) delta(i)).
 * Writes dq, dk, dv (dk/dv per KV head: the GQA group sum is taken inside),
 * dbias (nullable; requires a->bias; written in full, exactly 0 where
 * masked) and dsink (required iff sink_mode == ATTN_SINK_LEARNABLE, else must
 * be NULL; summed over every batch row and query row).  out_lo: nullable,
 * what attn_fwd wrote there (bf16 or fp16).  Results are deterministic (no
 * floating-point atomics): the same inputs give the same bits.
 * workspace: at least attn_bwd_workspace_size(a) bytes, 256-byte aligned. */
attn_status attn_bwd(const attn_args* a, const void* out, const void* out_lo, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, void* dbias, float* dsink, void* workspace, size_t workspace_bytes,
                     void* stream);

/* The same backward in three phases, for callers that time them
 * (attn_bwd == pre, then dkdv, then dq).  All three take the same arguments
 * and the same workspace, which carries the pre-pass results (segment runs,
 * delta = rowsum(dout * (out + out_lo)), sink-gradient partials) to the
 * other two and, with ATTN_DQ_DU_BLOCKS, the dU blocks that dkdv writes and
 * dq reads; so it must stay untouched between them and the phases must run
 * in that order (on one stream, or with the caller ordering them).
 *  - attn_bwd_pre:  segment runs, delta, dsink (required iff LEARNABLE) and,
 *                   except for bf16 with D = 128 or 256, the zeros of dbias
 *                   on the masked pairs (dbias nullable);
 *  - attn_bwd_dkdv: dk, dv and dbias on the visible pairs, and for bf16 with
 *                   D = 128 or 256 also its zeros (dbias nullable, complete
 *                   once attn_bwd_pre and attn_bwd_dkdv have both run; a
 *                   broadcast dbias is reduced at the end of this phase);
 *  - attn_bwd_dq:   dq. */
attn_status attn_bwd_pre(const attn_args* a, const void* out, const void* out_lo, const float* lse,
                         const void* dout, void* dbias, float* dsink, void* workspace, size_t workspace_bytes,
                         void* stream);
attn_status attn_bwd_dkdv(const attn_args* a, const float* lse, const void* dout, void* dk, void* dv,
                          void* dbias, void* workspace, size_t workspace_bytes, void* stream);
attn_status attn_bwd_dq(const attn_args* a, const float* lse, const void* dout, void* dq, void* workspace,
                        size_t workspace_bytes, void* stream);

/* attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace lives in a static device array of
 * 128 MiB inside the library, one per GPU (held until the process ends);
 * dq_mode ATTN_DQ_AUTO makes attn_bwd's choice where the whole workspace
 * then fits in it, else recomputes.  A problem whose workspace exceeds
 * 128 MiB is rejected with ATTN_UNSUPPORTED before anything is launched
 * (e.g. an explicit ATTN_DQ_DU_BLOCKS at B=4, Hq=32, S=4096).  The stream
 * must belong to the current device.  Outputs and their meaning are those of
 * attn_bwd, bit for bit when both resolve to the same dq_mode.
 * Every call on a GPU shares that GPU's array: calls that overlap in time on
 * one GPU (different streams or host threads without ordering between them)
 * race and give wrong results.  No call allocates or frees memory. */
attn_status attn_bwd_noalloc(const attn_args* a, const void* out, const void* out_lo, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, void* dbias, float* dsink,
                             void* stream);

/* Message for the last non-OK status on this thread ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_SOFTCAP_H */
