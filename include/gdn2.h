/*
 * gdn2.h -- C ABI of the MI355X (gfx950) Gated Delta Rule-2 library.
 *
 * The recurrence (Gated DeltaNet-2 pages: Spanish blog, gate table under
 * "Gated DeltaNet-2: La Solucion"; Korean summary, "method" steps 1-4;
 * Japanese article, "core" section), per sequence n, head h, token t:
 *
 *     S_t = (I - k_t (b_t (.) k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t (.) v_t)^T
 *     o_t = S_t^T q_t
 *
 * alpha_t in (0,1]^dk is the per-key-channel decay, applied before the edit;
 * b_t in [0,1]^dk the per-key-channel erase gate; w_t in [0,1]^dv the
 * per-value-channel write gate; S is the dk x dv fast-weight state.  The
 * erase gate multiplies the key that reads the prediction S'^T (b (.) k); the
 * edit is the rank-one k delta^T with delta = w (.) v - S'^T (b (.) k).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE memory (hipMalloc / torch CUDA tensors) unless a
 *    comment says otherwise; every tensor is contiguous, row-major, and owned
 *    by the caller.  The library allocates nothing and keeps no mutable
 *    global state; calls on different streams do not interfere.
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the null
 *    stream) and return without synchronising.  Results are valid once the
 *    stream has reached that point.
 *  - Argument errors are reported by the return code BEFORE anything is
 *    launched; nothing is printed.  GDN2_ERR_HIP reports a launch failure
 *    (hipGetLastError after the launches).  A fault inside a kernel surfaces
 *    at the caller's next synchronisation.
 *  - Preconditions that are documented but not checked on the device:
 *      0 < alpha <= 1;  finite inputs;  cu_seqlens non-decreasing, starting
 *      at 0 and ending at the packed token count;  for the bf16-input
 *      forward's fp16 operands: |v|, |S0| and the state stay below ~1e4 in
 *      magnitude, and the entries of q and k (of unit-norm vectors in the
 *      Gated DeltaNet-2 mixer) stay within 4 (the decayed tiles multiply
 *      them by factors up to 2^14).
 *  - Strong decay is checked on the device: the bf16-input forward factors
 *    the in-chunk decay around each 64-token chunk's midpoint into fp16
 *    operands, which holds while the decay over either half of a chunk stays
 *    within 2^-14 in every key channel (alpha >= 0.74 on average over the
 *    half).  A sequence (segment) with a chunk beyond that is recomputed
 *    token by token in fp32 by the same launch: correct, and far slower.
 *    The fp32-input chunked forward (dk = 64) keeps its factors in fp32; it
 *    needs the half-chunk decay to stay within 2^-126 (alpha >= 0.065 on
 *    average over 32 tokens), which is not checked.
 */
#ifndef GDN2_H
#define GDN2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. Token inputs share one type; the output may be the input
 * type or fp32; the state is always fp32. */
typedef enum { GDN2_F32 = 0, GDN2_BF16 = 1 } gdn2_dtype;

/* Gate forms (Spanish blog, "Jerarquia de Generalizacion"; Japanese article,
 * "core" section: the rule reduces to Kimi Delta Attention when the erase and
 * write gates collapse to one scalar per token, and to Gated DeltaNet when
 * the decay collapses to a scalar too).  A gate given "per head" is a
 * [rows, H] tensor in in_dtype -- one value per (token, head) -- that stands
 * for the same value in every channel; the other gates keep their full
 * per-channel shapes.  b and w may differ (the KDA and Gated DeltaNet cases
 * pass the same values for both).  Reading fewer gate bytes is the point:
 * the forward streams its inputs from HBM. */
typedef enum {
    GDN2_GATES_FULL = 0, /* alpha, b: [.., dk]; w: [.., dv]                      */
    GDN2_GATES_KDA = 1,  /* alpha: [.., dk]; b, w: per head                      */
    GDN2_GATES_GDN = 2   /* alpha, b, w: per head                                */
} gdn2_gates;

enum {
    GDN2_OK = 0,
    GDN2_ERR_INVALID_ARG = -1, /* null required pointer, bad sizes, bad combination */
    GDN2_ERR_UNSUPPORTED = -2, /* head sizes or dtypes with no kernel */
    GDN2_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required       */
    GDN2_ERR_HIP = -4          /* a launch failed                                 */
};

/* Library build identifier (monotone integer). */
int gdn2_version(void);

/* Static string for a status code. Never NULL. */
const char* gdn2_status_string(int status);

/* Bytes of device workspace gdn2_fwd (and gdn2_fwd_gates, any gate form)
 * needs for these sizes (0 is possible).  Arguments as for gdn2_fwd, with
 * num_seqs = B for a dense batch; returns 0 for invalid sizes too (gdn2_fwd
 * then rejects them).  Non-zero when there are fewer (sequence, head,
 * 64-column slab) workgroups than compute units and the sequences are long:
 * the forward then splits them into segments and keeps each segment's
 * state map and start state in the workspace (fp32, dk x (dv + dk) and
 * dk x dv per segment).  A packed batch (B == 1, num_seqs > 1) also keeps
 * int32[num_seqs] there. */
size_t gdn2_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                               int32_t num_seqs, int32_t in_dtype);

/*
 * gdn2_fwd -- chunkwise-WY forward over whole sequences (chunk of 64 tokens;
 * the in-chunk decay is folded into asymmetric erase factors: Spanish blog,
 * "Innovaciones Tecnicas" item 1; Korean summary, "main contributions" item 3
 * and "method" steps 3-4).  The result equals the token-by-token recurrence
 * above up to rounding and does not depend on the chunk size.
 *
 *   q, k, alpha, b : [B, T, H, dk]  in_dtype
 *   v, w           : [B, T, H, dv]  in_dtype
 *   S0             : [N, H, dk, dv] fp32 start state, or NULL (= zeros)
 *   o              : [B, T, H, dv]  out_dtype (in_dtype or GDN2_F32); must not
 *                    overlap an input, S0 or S_T (o equal to one of those
 *                    pointers: GDN2_ERR_INVALID_ARG)
 *   S_T            : [N, H, dk, dv] fp32 final state, or NULL (not written);
 *                    S_T == S0 is allowed (in-place state update)
 *   cu_seqlens     : NULL (then N = B and sequence n is batch row n), or a
 *                    DEVICE int32[num_seqs + 1] of packed offsets with B == 1
 *                    (then N = num_seqs and sequence n is tokens
 *                    cu_seqlens[n] .. cu_seqlens[n+1]-1; empty sequences are
 *                    allowed and leave S_T[n] = S0[n])
 *   dk, dv         : 64 or 128 each
 *   H              : H * max(dk, dv) < 2^24 (one 64-token chunk of a token
 *                    tensor is addressed with 32-bit byte offsets);
 *                    GDN2_ERR_INVALID_ARG otherwise
 *   in_dtype       : GDN2_BF16 or GDN2_F32
 *   workspace      : device buffer of >= gdn2_fwd_workspace_size(...) bytes
 *                    (may be NULL when that size is 0); contents need not be
 *                    initialised and are scratch after the call.
 *
 * Numerics: with bf16 inputs the in-chunk contractions run on fp16 MFMA
 * operands with fp32 accumulation and the state stays fp32; with fp32 inputs
 * every contraction runs on fp32 MFMA.  fp32 inputs at dk = 128 take the
 * token-serial recurrence instead (the chunked kernel's fp32 operand tiles
 * would exceed the 160 KB of LDS): all fp32, one step per token, far slower
 * per token than the chunked forward.
 */
int gdn2_fwd(const void* q, const void* k, const void* v, const void* alpha, const void* b,
             const void* w, int32_t in_dtype, const float* S0, void* o, int32_t out_dtype,
             float* S_T, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
             int32_t H, int32_t dk, int32_t dv, void* workspace, size_t workspace_bytes,
             void* stream);

/*
 * gdn2_fwd_gates -- gdn2_fwd with reduced gate forms (gdn2_gates above).
 * Arguments as for gdn2_fwd, except that under GDN2_GATES_KDA b and w, and
 * under GDN2_GATES_GDN alpha, b and w, are [B, T, H] tensors: one value per
 * (token, head), applied to every channel.  Same workspace size, results
 * equal to gdn2_fwd on the gates broadcast to full shape.  gates outside
 * gdn2_gates: GDN2_ERR_INVALID_ARG.  gdn2_fwd is this call with
 * GDN2_GATES_FULL.
 */
int gdn2_fwd_gates(const void* q, const void* k, const void* v, const void* alpha,
                   const void* b, const void* w, int32_t gates, int32_t in_dtype, const float* S0,
                   void* o, int32_t out_dtype, float* S_T, const int32_t* cu_seqlens,
                   int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn2_decode -- one recurrent step for N sequences (constant-memory decode:
 * Spanish blog, "Por Que Es Importante" item 1; Korean summary, "results"
 * item 2).  The state is read once and written once:
 *     S' = Diag(alpha) S,  r = S'^T (b (.) k),  p = S'^T q,  delta = w (.) v - r,
 *     S <- S' + k delta^T,  o = p + (q . k) delta   (= S_new^T q).
 *
 *   q, k, alpha, b : [N, H, dk]  in_dtype      v, w : [N, H, dv]  in_dtype
 *   S              : [N, H, dk, dv] fp32, updated in place
 *   o              : [N, H, dv] out_dtype (in_dtype or GDN2_F32); must not
 *                    overlap an input or S (o equal to one of those pointers:
 *                    GDN2_ERR_INVALID_ARG)
 *   dk, dv         : 64 or 128 each
 * All arithmetic is fp32.
 */
int gdn2_decode(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                const void* w, int32_t in_dtype, float* S, void* o, int32_t out_dtype, int32_t N,
                int32_t H, int32_t dk, int32_t dv, void* stream);

/*
 * gdn2_decode_gates -- gdn2_decode with reduced gate forms: under
 * GDN2_GATES_KDA b and w, under GDN2_GATES_GDN alpha, b and w, are [N, H]
 * tensors (one value per sequence and head, applied to every channel).
 * gates outside gdn2_gates: GDN2_ERR_INVALID_ARG.  gdn2_decode is this call
 * with GDN2_GATES_FULL.
 */
int gdn2_decode_gates(const void* q, const void* k, const void* v, const void* alpha,
                      const void* b, const void* w, int32_t gates, int32_t in_dtype, float* S,
                      void* o, int32_t out_dtype, int32_t N, int32_t H, int32_t dk, int32_t dv,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H */
