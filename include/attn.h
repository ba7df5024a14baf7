/*
 * attn.h -- C ABI of the fused scaled dot-product attention forward pass for
 * AMD Instinct MI355X (gfx950).
 *
 * Operation (codelab "Accelerate attention on GPU with cuDNN and
 * TransformerEngine", intro "How attention works" and section 4; article
 * "Self-attention, CUDA kernels and FlashAttention", sections 1 and 3):
 *
 *   O[b,h,i,:] = sum_j softmax_j( scale * Q[b,h,i,:] . K[b,hk,j,:] ) * V[b,hk,j,:]
 *   lse[b,h,i] = ln sum_j exp( scale * Q[b,h,i,:] . K[b,hk,j,:] )
 *
 * over the allowed keys j: all of [0, Sk), or j <= i + (Sk - Sq) with the
 * causal (lower-triangular) mask of the codelab's section 7, the queries
 * being the last Sq of the Sk positions (Sq == Sk is self-attention; Sq < Sk
 * is new queries against a longer key sequence, as with a KV cache). Query head h reads KV
 * head hk = h / (Hq / Hkv): consecutive groups of query heads share one KV
 * head (MHA when Hkv == Hq, GQA, MQA when Hkv == 1; codelab section 9).
 * The computation is fused in the FlashAttention manner (article section 3):
 * score tiles live only on chip, so no Sq x Sk matrix is written to memory;
 * lse is the small per-row statistic that manner keeps for a backward pass.
 *
 * Layouts (dense, row-major; attn_fwd_strided takes strided q, k, v, o):
 *   q, o  : [B, Hq,  Sq, d]
 *   k, v  : [B, Hkv, Sk, d]
 *   lse   : [B, Hq,  Sq] float32, natural-log units (may be NULL)
 *
 * Ownership and execution:
 *   - every pointer is a DEVICE pointer owned by the caller; the library
 *     allocates no memory, keeps no state, and is safe to call from several
 *     host threads;
 *   - work is enqueued on `stream` (NULL = the null stream) and the call
 *     returns without waiting; errors of the kernel itself surface on the
 *     stream, as for any HIP launch;
 *   - every element of o (and of lse when non-NULL) is written;
 *   - outputs must not overlap inputs; base pointers must be 16-byte aligned.
 *
 * Errors are returned, never hidden: an unsupported request is rejected
 * before anything is enqueued and nothing falls back to another path
 * (the codelab's section 6 makes the same choice for its fused backend).
 */
#ifndef SDPA18_ATTN_H
#define SDPA18_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v. Output o is f32 for ATTN_F32 and bf16 otherwise. */
typedef enum {
  ATTN_F32 = 0,      /* IEEE binary32 in, binary32 out                          */
  ATTN_BF16 = 1,     /* bfloat16 in, bfloat16 out (RNE)                          */
  ATTN_FP8_E4M3 = 2  /* OCP fp8 e4m3fn codes in (unit descales), bfloat16 out    */
} attn_dtype_t;

/* Status codes: 0 is success, every error is negative. */
enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,          /* a required pointer is NULL (q, k, v, o; see attn_bwd) */
  ATTN_ERR_SHAPE = -2,         /* a size is < 1, or the problem exceeds 32-bit indexing */
  ATTN_ERR_HEADS = -3,         /* Hq is not a multiple of Hkv                           */
  ATTN_ERR_HEADDIM = -4,       /* d not in {32, 64, 128} ({64, 128}: split-KV, backward) */
  ATTN_ERR_CAUSAL_SHAPE = -5,  /* causal requested with Sq > Sk                         */
  ATTN_ERR_DTYPE = -6,         /* dtype is not an attn_dtype_t value                    */
  ATTN_ERR_SCALE = -7,         /* scale or a descale is not finite and > 0              */
  ATTN_ERR_ALIGN = -8,         /* a base pointer is not 16-byte aligned                 */
  ATTN_ERR_LAUNCH = -9,        /* the HIP runtime rejected the launch or a device query */
  ATTN_ERR_WORKSPACE = -10,    /* split-KV workspace missing, misaligned or too small   */
  ATTN_ERR_SPLITS = -11,       /* num_splits outside [0, 128]                           */
  ATTN_ERR_STRIDE = -12,       /* attn_fwd_strided: unusable strides (see there)        */
  ATTN_ERR_SCRATCH = -13       /* attn_fwd_splitkv_noalloc: needs more than ATTN_SCRATCH_BYTES */
};

/*
 * attn_fwd -- fused attention forward.
 *
 *   q, k, v  device inputs of element type `dtype`, layouts above.
 *   o        device output: float32 for ATTN_F32, bfloat16 otherwise.
 *   lse      device float32 [B, Hq, Sq] or NULL to skip the statistic.
 *   B, Hq, Hkv, Sq, Sk, d   sizes; Hq % Hkv == 0; d in {32, 64, 128} (the
 *            codelab's closing next steps try head dimensions 32, 64 and 128);
 *            causal requires Sq <= Sk.
 *   scale    multiplier of the dot products, finite and > 0 (the pages use
 *            1/sqrt(d)).
 *   causal   0 = every key visible; nonzero = key j visible to query i iff
 *            j <= i + (Sk - Sq).
 *   dtype    attn_dtype_t; ATTN_FP8_E4M3 here means all descales are 1.
 *   stream   HIP stream to enqueue on.
 *
 * Returns ATTN_OK or a negative status (see above).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int d,
             float scale, int causal, int dtype, hipStream_t stream);

/*
 * attn_fwd_fp8 -- fused attention forward on fp8 e4m3fn inputs with
 * per-tensor scales (codelab section 10: E4M3 forward format, per-tensor amax
 * scaling). The real value of an input element is code * descale_x, with
 * descale_x = amax(|x|) / 448 for per-tensor amax quantisation. Q.K^T runs on
 * fp8 matrix cores with fp32 accumulation; the descales of Q and K fold into
 * the softmax scale and descale_v into the epilogue.
 *
 *   q8, k8, v8  device uint8 e4m3fn codes, layouts as attn_fwd.
 *   o_bf16      device bfloat16 output [B, Hq, Sq, d].
 *   lse         as attn_fwd (of the dequantised scores), or NULL.
 *   descale_q, descale_k, descale_v  finite and > 0.
 *   Other arguments and the return value as attn_fwd.
 */
int attn_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o_bf16, float* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                 float descale_q, float descale_k, float descale_v, hipStream_t stream);

/*
 * attn_fwd_strided -- attn_fwd / attn_fwd_fp8 on strided tensors, so that the
 * codelab's own (B, T, N, H) arrays ("Accelerate attention on GPU with cuDNN
 * and TransformerEngine", sections 3 and 4: batch, sequence, heads, head
 * dimension) are read and written in place, without a permute.
 *
 *   strides  12 element strides: {batch, head, position} of q, then k, v, o.
 *            Element [b, h, i, c] of q sits at q + b*s[0] + h*s[1] + i*s[2] + c;
 *            the d elements of one position are contiguous. The dense layout
 *            of attn_fwd is {Hq*Sq*d, Sq*d, d} for q and o; the codelab's
 *            (B, T, N, H) is {T*N*H, H, N*H}.
 *            Every stride must be >= 0, the position stride >= d, each stride
 *            in bytes a multiple of 16, and one head's rows must span less
 *            than 2 GiB; otherwise ATTN_ERR_STRIDE. Distinct (b, h, i) of o
 *            must not overlap (not checked).
 *   dtype    as attn_fwd; for ATTN_FP8_E4M3 descale_q/k/v are the per-tensor
 *            descales of attn_fwd_fp8, for the other dtypes they must be 1.
 *   lse      dense [B, Hq, Sq] as in attn_fwd.
 *   Other arguments and the return value as attn_fwd.
 */
int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d, const int64_t* strides,
                     float scale, int causal, int dtype,
                     float descale_q, float descale_k, float descale_v, hipStream_t stream);

/*
 * attn_fwd_splitkv -- the same operation as attn_fwd, computed for few
 * queries against a long key sequence (decoding against a KV cache: Sq of 1
 * to a few dozen, Sk in the thousands; the codelab's section 9 shares KV heads
 * between query heads, and its closing next steps point at such shapes). The
 * rows of the G = Hq / Hkv query heads that share a KV head are computed
 * together, and the keys of each KV head are cut into num_splits chunks that
 * run in parallel. Each chunk yields a normalised partial output and its
 * log-sum-exp; a second kernel merges them exactly (softmax over the union of
 * chunks: weights exp(lse_s - max lse), the rescaling step of the online
 * softmax in the article's section 3). Results agree with attn_fwd up to
 * rounding.
 *
 *   q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, stream  as attn_fwd,
 *                except d in {64, 128}.
 *   dtype        ATTN_BF16 only (ATTN_ERR_DTYPE otherwise).
 *   num_splits   0 = the library's choice (enough chunks to fill the GPU, at
 *                least 256 keys each), else at most 128 chunks; a chunk holds
 *                a multiple of 32 keys, so fewer may run (see the plan call).
 *   workspace    device memory owned by the caller, 16-byte aligned, of at
 *                least the size attn_fwd_splitkv_plan reports for the same
 *                sizes and num_splits; may be NULL when that size is 0 (one
 *                chunk). It holds fp32 partial outputs [B*Hq*Sq][splits][d]
 *                then their base-2 log-sum-exps [B*Hq*Sq][splits]; contents
 *                on entry are ignored and on return are unspecified. Two
 *                calls in flight at once need two workspaces.
 *
 * Returns ATTN_OK or a negative status; ATTN_ERR_WORKSPACE if the workspace
 * is missing, misaligned or too small, ATTN_ERR_SPLITS if num_splits is
 * outside [0, 128].
 */
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d,
                     float scale, int causal, int dtype, int num_splits,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_fwd_splitkv_plan -- host-only query: the number of key chunks
 * attn_fwd_splitkv will run for these sizes and num_splits (*splits_used)
 * and the workspace bytes it needs (*workspace_bytes, 0 for one chunk).
 * Either output pointer may be NULL. Enqueues nothing. Returns ATTN_OK or the
 * status attn_fwd_splitkv would return for these sizes.
 */
int attn_fwd_splitkv_plan(int B, int Hq, int Hkv, int Sq, int Sk, int d, int num_splits,
                          int* splits_used, size_t* workspace_bytes);

/*
 * attn_fwd_splitkv_noalloc -- attn_fwd_splitkv without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments (minus workspace), same kernels, bit-identical results.
 *
 * The key chunks' partial outputs and log-sum-exps go to a static device
 * array inside the library, ATTN_SCRATCH_BYTES (16 MiB) per GPU, held by each
 * GPU the library runs on until the process ends. Nothing is allocated: no
 * hipMalloc, no hipFree, no allocating library call. The array's device
 * address is looked up on the first call on each device (the current device;
 * `stream` must belong to it). The chunk kernel writes every entry the merge
 * kernel reads, so no call depends on what an earlier call left there.
 *
 * Every call on one GPU shares that GPU's array: two calls whose work can
 * overlap on one GPU (different streams, or host threads without ordering)
 * race on it and may return wrong results. Calls on one stream are ordered
 * and safe.
 *
 * Returns ATTN_OK, ATTN_ERR_SCRATCH when attn_fwd_splitkv_plan reports more
 * than ATTN_SCRATCH_BYTES of workspace for these sizes and num_splits
 * (nothing is enqueued), or the other statuses of attn_fwd_splitkv.
 */
#define ATTN_SCRATCH_BYTES ((size_t)16 << 20)
int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int Hq, int Hkv, int Sq, int Sk, int d,
                             float scale, int causal, int dtype, int num_splits, hipStream_t stream);

/*
 * attn_bwd -- gradients of the attention forward (the backward pass the
 * article "Self-attention, CUDA kernels and FlashAttention", section 3,
 * describes: the attention weights are recomputed tile by tile from the
 * forward's per-row log-sum-exp instead of being stored). For a loss L with
 * dout = dL/dO:
 *
 *   P = exp(scale Q K^T - lse)  (masked pairs 0)    dV = P^T dout
 *   dS = P * (dout V^T - rowsum(dout * O))          dQ = scale dS K
 *   dK = scale dS^T Q
 *
 * summed over the query heads that share a KV head (GQA/MQA). The mask, the
 * head mapping and the layouts are those of attn_fwd.
 *
 *   q, k, v   the forward's inputs; o, lse its outputs (lse is required);
 *   dout      dL/dO, layout of o;
 *   dq        output, layout of q; dk, dv outputs, layout of k / v. Every
 *             element is written (a KV head's gradient is the sum over its
 *             query heads, computed without atomics);
 *   dtype     ATTN_BF16: bf16 q, k, v, o, dout, dq, dk, dv, d in {64, 128};
 *             ATTN_F32: fp32 q, k, v, o, dout, dq, dk, dv, d in {32, 64, 128}
 *             (fp32 matrix cores throughout); lse is fp32 in both;
 *   workspace device memory owned by the caller, 16-byte aligned, at least
 *             attn_bwd_workspace_size bytes (that size serves both dtypes):
 *             2*B*Hq*Sq floats (the per-row rowsum(dout * O), then
 *             lse * log2(e)), and, for bf16 when the query heads of a KV head
 *             are split into s > 1 subsets (groups of 8 or more heads on grids
 *             under 512 dK/dV workgroups, e.g. MQA), from the next 16-byte
 *             boundary the fp32 partial dK and dV of every subset
 *             (2*s*B*Hkv*Sk*d floats), summed in subset order; contents on
 *             entry ignored, unspecified on return; two calls in flight need
 *             two workspaces.
 *   Other arguments as attn_fwd.
 *
 * Returns ATTN_OK or a negative status: ATTN_ERR_NULL if any of q, k, v, o,
 * dout, lse, dq, dk, dv is NULL, ATTN_ERR_WORKSPACE for a missing, misaligned
 * or short workspace, the other codes as attn_fwd.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Sq, int Sk, int d,
             float scale, int causal, int dtype,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* attn_bwd_workspace_size -- host-only: the workspace bytes attn_bwd needs
 * for these sizes (*workspace_bytes, may be NULL), for either dtype. Returns
 * ATTN_OK or the size error attn_bwd would return. */
int attn_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int d, size_t* workspace_bytes);

/*
 * attn_bwd_fp8 -- attn_bwd for fp8 inputs in the codelab's fp8 recipe
 * (section 10: E4M3 for the forward tensors, E5M2 for the gradients, each
 * with a per-tensor scale): the same gradients, of the real values
 *
 *   Q = descale_q * q8,  K = descale_k * k8,  V = descale_v * v8,
 *   dO = descale_do * dout8.
 *
 *   q8, k8, v8  device uint8 e4m3fn codes, layouts as attn_fwd;
 *   o           device bfloat16 [B, Hq, Sq, d], the output of attn_fwd_fp8
 *               for these inputs; lse its fp32 log-sum-exp (required);
 *   dout8       device uint8 e5m2 codes of dL/dO, layout of o;
 *   dq, dk, dv  device bfloat16 outputs (real values), layouts of q / k / v;
 *   descale_*   finite and > 0;
 *   d           64 or 128;
 *   workspace   device memory owned by the caller, 16-byte aligned, at least
 *               attn_bwd_fp8_workspace_size bytes: attn_bwd's workspace, then
 *               bf16 copies of q8, dout8, k8 and v8 (each code widened, which
 *               is exact); contents on entry ignored, unspecified on return.
 *   Other arguments as attn_bwd.
 *
 * The codes are widened to bf16 and the products run on bf16 matrix cores
 * with fp32 accumulation; the descales fold into the softmax scale and the
 * output factors. Returns as attn_bwd.
 */
int attn_bwd_fp8(const void* q8, const void* k8, const void* v8, const void* o, const void* dout8,
                 const float* lse, void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                 float descale_q, float descale_k, float descale_v, float descale_do,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* attn_bwd_fp8_workspace_size -- host-only: the workspace bytes attn_bwd_fp8
 * needs for these sizes (*workspace_bytes, may be NULL). Returns ATTN_OK or
 * the size error attn_bwd_fp8 would return. */
int attn_bwd_fp8_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int d, size_t* workspace_bytes);

/* attn_strerror -- static, NUL-terminated text for a status code (never NULL). */
const char* attn_strerror(int status);

/* attn_version -- ABI version of this library (major * 10000 + minor * 100 + patch). */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA18_ATTN_H */
