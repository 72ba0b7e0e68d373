/*
 * fa.h -- C ABI of libfa, exact tiled attention for AMD Instinct MI355X (gfx950).
 *
 * The operation (all entry points): exact attention
 *     O = softmax(scale * Q K^T) V,   lse_i = ln sum_j exp(scale * q_i . k_j),
 * computed as tiled attention with an online softmax (running row max m,
 * running sum l, partial O rescaled by exp(m_old - m_new)), never writing the
 * score matrix S or the weight matrix P to memory.
 *   - Definition: "Flash Attention Mechanics: How Tiled Attention Fits in SRAM",
 *     section "Why Standard Attention Is Memory-Bound"; "Why is standard
 *     attention memory-bound, and how does FlashAttention fix it?", "Step 1".
 *   - Tiling and the online softmax: the same Mechanics page, section "The
 *     Tiling Algorithm"; the memory-bound page, "Step 3" and "What is online
 *     softmax?".
 *   - Causal tile skipping and decode: "FlashAttention HBM bytes, one head, 8K",
 *     section "What interviewers probe next".
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library never
 *     frees them and keeps no reference after the call returns.
 *   - Every tensor of a call, its workspace and `stream` belong to one GPU, which
 *     must be the calling thread's current HIP device: launch planning (key
 *     splits, workspace sizes) reads that device's compute-unit count, and
 *     fa_fwd's temporary buffer comes from its memory pool.
 *   - BF16 tensors are IEEE bfloat16 bit patterns; every tensor is contiguous
 *     (row-major in the order its shape is written) and 16-byte aligned.
 *   - Argument checks run on the host before any launch or allocation (the
 *     only HIP call before them is a cached compute-unit-count query). On
 *     failure the call returns a negative fa_status and launches nothing;
 *     outputs are untouched.
 *   - Work is enqueued asynchronously on `stream` (NULL = the null stream). A
 *     launch failure returns FA_ERR_LAUNCH; faults during execution surface at
 *     the caller's next synchronisation.
 *   - GQA: query head h reads KV head h / (Hq / Hkv).
 *   - scale is used exactly as given (any finite value, including 0 and
 *     negative); the usual choice is 1/sqrt(d).
 *   - The functions are thread-safe; concurrent calls on different streams do
 *     not share memory unless the caller passes the same buffers (except
 *     fa_fwd_noalloc, whose calls on one GPU share its static scratch).
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same objects as hipStream_t and hipEvent_t, declared without the HIP headers. */
struct ihipStream_t;
typedef struct ihipStream_t* fa_stream_t;
struct ihipEvent_t;
typedef struct ihipEvent_t* fa_event_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,      /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,     /* a size is <= 0, too large (N or L above 2^30, B*Hq*N above 2^31 - 1,
                            a grid beyond 2^31 - 1 work-groups), or num_splits out of range */
  FA_ERR_HEAD_DIM = -3,  /* d is not 64 or 128 */
  FA_ERR_GQA = -4,       /* Hq is not a multiple of Hkv */
  FA_ERR_ALIGN = -5,     /* a tensor pointer is not 16-byte aligned (lse: 4-byte) */
  FA_ERR_WORKSPACE = -6, /* workspace NULL or smaller than the queried size */
  FA_ERR_LAUNCH = -7,    /* a HIP launch or allocation failed */
  FA_ERR_ARG = -8,       /* causal not 0/1, or a scale (factor) not finite */
  FA_ERR_SCRATCH = -9    /* fa_fwd_noalloc: the key-split partials exceed its static scratch */
} fa_status;

/*
 * fa_fwd -- attention forward pass (prefill).
 *
 *   q   [B, Hq,  N, d] bf16   queries
 *   k   [B, Hkv, N, d] bf16   keys
 *   v   [B, Hkv, N, d] bf16   values
 *   o   [B, Hq,  N, d] bf16   output, written once, rounded to nearest even
 *   lse [B, Hq,  N]    fp32   natural-log logsumexp of each row's scaled scores
 *   causal: 0 = every key visible; 1 = key j visible to query i iff j <= i.
 *
 * d must be 64 or 128. One kernel launch per call, except when the query
 * blocks (128 or 256 rows) would leave the GPU's compute units idle: then the
 * keys of every query block are split across work-groups (at least 512 keys
 * per split; as many work-groups as fit on the compute units at once), each
 * writing its normalised partial output (BF16, rounded to nearest even) and
 * logsumexp (FP32), and a second launch merges them with the log-sum-exp
 * combine. That path takes a stream-ordered temporary buffer of
 * B*Hq*N*splits*(2d+4) bytes from the device's default memory pool
 * (hipMallocAsync / hipFreeAsync on `stream`) and returns FA_ERR_LAUNCH if the
 * pool cannot supply it.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           fa_stream_t stream);

/*
 * fa_fwd_workspace_bytes -- bytes of caller-provided workspace that fa_fwd_ws
 * needs for these sizes on the current device: 0 when the forward runs as one
 * launch, else the key-split partials (BF16 [B*Hq*N, splits, d] followed by
 * FP32 [B*Hq*N, splits]) rounded up to 256 bytes. Returns 0 for invalid sizes.
 */
size_t fa_fwd_workspace_bytes(int B, int Hq, int N, int d);

/*
 * fa_fwd_ws -- fa_fwd with a caller-owned workspace instead of the
 * stream-ordered temporary buffer: same operation, arguments and layouts, plus
 * workspace / workspace_bytes (device memory, 16-byte aligned, at least
 * fa_fwd_workspace_bytes(B, Hq, N, d); may be NULL when that is 0; contents on
 * entry are ignored). Calls sharing a workspace must be ordered.
 */
int fa_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
              void* workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * fa_fwd_ws_timed -- fa_fwd_ws that also records `after_attention` (a HIP
 * event created by the caller) on `stream` right after the attention kernel's
 * launch and before the key-split merge (the end of the call when it has no
 * merge), so that the caller can time the attention kernel alone with events.
 * Same operation, arguments, results and errors as fa_fwd_ws; after_attention
 * must not be NULL (FA_ERR_NULL), and a failed record returns FA_ERR_LAUNCH.
 */
int fa_fwd_ws_timed(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                    void* workspace, size_t workspace_bytes, fa_stream_t stream,
                    fa_event_t after_attention);

/*
 * fa_fwd_noalloc -- fa_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): same operation, arguments, layouts and kernels, but the key-split
 * partials go to a static device array of fa_fwd_noalloc_max_scratch_bytes()
 * bytes (34 MiB) that the library holds on each GPU it runs on until the process
 * ends. The call itself allocates nothing; its first call on a device only looks
 * up that device's copy of the array (hipGetSymbolAddress).
 *
 * Shapes whose partials (fa_fwd_workspace_bytes-sized; 17.0 MB for one head of
 * 8192 keys at d = 128) exceed the array return FA_ERR_SCRATCH before any
 * launch. On a 256-CU GPU no valid shape does. Every call on one GPU shares
 * that GPU's array: calls that may overlap on one GPU (different streams,
 * different host threads) race and must be ordered by the caller. Each call
 * writes every partial it reads, so the array keeps the last call's contents
 * and needs no clearing. A call records only kernel launches (no memset, no
 * allocation), so it may be captured in a HIP graph once one call on that
 * device (outside the capture) has looked up the array's address.
 */
int fa_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   fa_stream_t stream);

/* Size in bytes of fa_fwd_noalloc's static per-GPU scratch array. */
size_t fa_fwd_noalloc_max_scratch_bytes(void);

/*
 * fa_fwd_fp8 -- attention forward pass on FP8 inputs ("Why is standard
 * attention memory-bound, and how does FlashAttention fix it?", follow-up
 * "What does FlashAttention-2 change?": the third version adds 8-bit floating
 * point low precision). Same operation as fa_fwd on the dequantised inputs:
 *
 *   q   [B, Hq,  N, d] uint8  OCP FP8 E4M3 codes; the query values are q_scale * Q
 *   k   [B, Hkv, N, d] uint8  E4M3 codes; keys k_scale * K
 *   v   [B, Hkv, N, d] uint8  E4M3 codes; values v_scale * V
 *   o   [B, Hq,  N, d] bf16   output, rounded to nearest even
 *   lse [B, Hq,  N]    fp32   natural-log logsumexp of scale * q.k (dequantised)
 *
 * d must be 64 or 128 (FA_ERR_HEAD_DIM otherwise). q_scale, k_scale, v_scale and
 * scale * q_scale * k_scale must be finite (FA_ERR_ARG otherwise); any sign.
 * Arithmetic: Q.K products exact, accumulated by the FP8 matrix cores; the
 * weights 2^(t - m + 6) are rounded to E4M3 (relative error <= 2^-4) for the
 * P V product while the row sums use their FP32 values; O and lse otherwise
 * as fa_fwd. Key splits, their temporary buffer and the errors are those of
 * fa_fwd (the workspace size is fa_fwd_workspace_bytes(B, Hq, N, d)).
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale, float v_scale,
               void* o, float* lse, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
               fa_stream_t stream);

/* fa_fwd_fp8_ws -- fa_fwd_fp8 with a caller-owned workspace, as fa_fwd_ws. */
int fa_fwd_fp8_ws(const void* q, const void* k, const void* v, float q_scale, float k_scale, float v_scale,
                  void* o, float* lse, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                  void* workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * fa_decode_workspace_bytes -- size of the caller-provided workspace that
 * fa_decode needs for these sizes: FP32 partial outputs [B, Hq, S, d] and
 * partial logsumexps [B, Hq, S], S = number of non-empty chunks. Returns 0 for
 * invalid sizes.
 */
size_t fa_decode_workspace_bytes(int B, int Hq, int L, int d, int num_splits);

/*
 * fa_decode -- split-KV decode: one query token per (sequence, query head)
 * against a KV cache of L keys ("What interviewers probe next", decode; "Does
 * FlashAttention help when generating one token at a time?").
 *
 *   q   [B, Hq,  1, d] bf16
 *   k   [B, Hkv, L, d] bf16
 *   v   [B, Hkv, L, d] bf16
 *   o   [B, Hq,  1, d] bf16
 *   lse [B, Hq]        fp32 (natural log)
 *   workspace: device buffer of at least fa_decode_workspace_bytes(...) bytes,
 *   16-byte aligned, owned by the caller; its contents on entry are ignored.
 *
 * The L keys are cut into chunks of ceil(L / num_splits) keys (1 <= num_splits
 * <= L). One launch computes, per (sequence, KV head, chunk), the chunk's
 * normalised partial output and logsumexp for every query head of the group,
 * reading each K/V byte once; a second launch merges the chunks with the
 * log-sum-exp combine. Two calls that share a workspace must be ordered.
 */
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int Hq, int Hkv, int L, int d, int num_splits, float scale,
              void* workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * fa_decode_varlen -- fa_decode over a padded KV cache whose sequences have
 * their own lengths (a batch of real KV caches). Sequence b attends to keys
 * 0 .. len_b - 1 of its cache rows, len_b = seq_lens[b] clamped to [0, L];
 * keys past len_b are never read (they may hold anything). A sequence with
 * len_b = 0 gets O = 0 and lse = -inf.
 *
 *   seq_lens [B] int32, device memory, 4-byte aligned; read by the kernels,
 *            so it cannot be validated on the host.
 *   Every other argument, the layouts and the workspace
 *   (fa_decode_workspace_bytes(B, Hq, L, d, num_splits)) are those of
 *   fa_decode. Each sequence's own len_b keys are cut into chunks of
 *   max(ceil(len_b / S), 128) keys (at most the S that fa_decode would use
 *   for L), so the work of a sequence spreads over its work-groups; chunks
 *   past len_b are empty and take no part in the merge.
 */
int fa_decode_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* seq_lens,
                     int B, int Hq, int Hkv, int L, int d, int num_splits, float scale,
                     void* workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * fa_bwd_workspace_bytes -- bytes of device workspace fa_bwd needs: two FP32
 * values per query row (lse in base 2 and -delta, delta = rowsum(dO O)), each head's
 * rows padded to a multiple of 64. 0 for invalid sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int N, int d);

/*
 * fa_bwd -- backward pass of fa_fwd: given the upstream gradient dO, the
 * gradients dQ, dK, dV of O = softmax(scale Q K^T) V (causal: key j visible to
 * query i iff j <= i), recomputing the scores tile by tile from Q, K and the
 * forward's lse ("Why is standard attention memory-bound, and how does
 * FlashAttention fix it?", "Step 4: The result is exact, and the backward
 * pass recomputes"). For GQA a KV head's dK, dV sum over the query heads that
 * read it.
 *
 *   q, o, dout, dq [B, Hq,  N, d] bf16;  k, v, dk, dv [B, Hkv, N, d] bf16
 *   lse            [B, Hq,  N]    fp32, natural log, as fa_fwd wrote it
 *   d = 64 or 128 (FA_ERR_HEAD_DIM otherwise).
 *   workspace: device, 16-byte aligned, at least fa_bwd_workspace_bytes(B, Hq,
 *   N, d) bytes, owned by the caller; contents on entry are ignored. Calls
 *   sharing a workspace must be ordered.
 *
 * Every gradient is written once (no accumulation into the outputs). Three
 * launches on `stream`: a row pass, dK/dV, dQ. Argument errors as fa_fwd.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           void* workspace, size_t workspace_bytes, fa_stream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
