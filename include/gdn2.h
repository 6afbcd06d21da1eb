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
 *      at 0 and ending at the packed token count.
 *  - The numeric range of the chunked forward is checked on the device.  The
 *    bf16-input forward factors the in-chunk decay around each 64-token
 *    chunk's midpoint into fp16 MFMA operands.  A chunk is in range when, in
 *    every key channel, the decay over either half of the chunk is at least
 *    2^-14 (alpha >= 0.74 on average over the half), the entries of q and k
 *    are at most 16 and at most 2^15 times that half-chunk decay, and every
 *    value the kernel converts to fp16 (w (.) v, the decayed state, the WY
 *    solution Delta, the inverses of A's diagonal blocks) is at most 2^15 in
 *    magnitude.  A sequence (segment) with a chunk out of range, or with a
 *    non-finite value in one, is recomputed token by token in fp32 by the
 *    same launch: correct, and far slower.  The fp32-input chunked forward
 *    (dk = 64) keeps its factors in fp32 and falls back the same way when a
 *    half-chunk decay drops below 2^-126.
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

/* Readings of the erase gate (Spanish blog, gate table under "Gated
 * DeltaNet-2: La Solucion": b_t acts on the key side; the pages do not say
 * on which factor of the erase product).  GDN2_ERASE_READ, the reading of
 * every other call: b gates the key that reads the prediction,
 *     S_t = (I - k_t (b_t (.) k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t (.) v_t)^T.
 * GDN2_ERASE_ROWS: b gates the erased rows,
 *     S_t = (I - (b_t (.) k_t) k_t^T) Diag(alpha_t) S_{t-1} + k_t (w_t (.) v_t)^T.
 * Both reduce to Kimi Delta Attention and Gated DeltaNet when b is a scalar
 * times 1.  The kernels take the reading as a compile-time switch. */
typedef enum { GDN2_ERASE_READ = 0, GDN2_ERASE_ROWS = 1 } gdn2_erase;

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
 * per token than the chunked forward; long sequences with few (sequence,
 * head) pairs are split into segments there too (see gdn2_fwd_ex).
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
 * gdn2_bwd -- gate-aware chunked backward of gdn2_fwd (Spanish blog,
 * "Innovaciones Tecnicas" item 2: the gradient flows through both the erase
 * and the write gate; Korean summary, "method", closing paragraph: no memory
 * beyond the chunk states).  For the loss
 *     L = sum_t <dout_t, o_t> + <dS_T, S_T>
 * of the forward with the same inputs, it writes dL/dq, dL/dk, dL/dv,
 * dL/dalpha, dL/db, dL/dw and dL/dS0 -- the exact gradients of the token
 * recurrence up to rounding, whatever the chunking.
 *
 *   q .. w, S0, cu_seqlens, num_seqs, B, T, H, dk, dv, in_dtype : as gdn2_fwd
 *                    (gate form: per channel only)
 *   dout           : [B, T, H, dv] in_dtype, the gradient of o
 *   dS_T           : [N, H, dk, dv] fp32 gradient of S_T, or NULL (= zeros)
 *   dq, dk, dalpha, db : [B, T, H, dk] grad_dtype;  dv, dw : [B, T, H, dv]
 *                    grad_dtype (in_dtype or GDN2_F32)
 *   dS0            : [N, H, dk, dv] fp32, or NULL (not written)
 *   workspace      : device buffer of >= gdn2_bwd_workspace_size(...) bytes
 *                    (contents need not be initialised; scratch afterwards)
 * No gradient buffer may equal an input or another gradient buffer
 * (GDN2_ERR_INVALID_ARG); other errors as for gdn2_fwd.
 *
 * Method: the forward runs again in a mode that stores every chunk's start
 * state; a per-chunk pass rebuilds the chunk's WY factors; a reverse walk
 * over the chunks carries dL/dS (one workgroup per sequence, head and 64
 * value columns); a per-chunk pass forms the gradients of q, k, b, alpha.
 * All backward arithmetic is fp32 (the products on fp32 MFMA).  The
 * half-chunk decay must stay at or above 2^-126 in every key channel
 * (alpha >= 0.065 on average over 32 tokens); this is not checked.
 */
size_t gdn2_bwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                               int32_t num_seqs, int32_t in_dtype);
int gdn2_bwd(const void* q, const void* k, const void* v, const void* alpha, const void* b,
             const void* w, int32_t in_dtype, const float* S0, const void* dout,
             const float* dS_T, void* dq, void* dk, void* dv, void* dalpha, void* db, void* dw,
             int32_t grad_dtype, float* dS0, const int32_t* cu_seqlens, int32_t num_seqs,
             int32_t B, int32_t T, int32_t H, int32_t dk_, int32_t dv_, void* workspace,
             size_t workspace_bytes, void* stream);

/*
 * gdn2_prologue -- the token mixer's elementwise steps in front of the
 * recurrence (Japanese article, "architecture and benchmarks", paragraph 1:
 * q and k through a short causal convolution, SiLU and an L2 normalisation
 * per head-token; v through a short convolution and SiLU; the three gates
 * through a sigmoid), after the projections, in one pass over HBM:
 *     q = L2norm(SiLU(conv(xq))),  k = L2norm(SiLU(conv(xk))),  v = SiLU(conv(xv)),
 *     alpha = sigmoid(ga),  b = sigmoid(gb),  w = sigmoid(gw)
 * conv is the depthwise causal convolution of width conv_width (1..4) along
 * each sequence: y_t[c] = sum_j W[c][j] x_{t - conv_width + 1 + j}[c], with
 * tokens before the sequence's first as zero.  L2norm(y) = y / sqrt(sum y^2
 * + l2_eps) over the dk channels of a (token, head).
 *
 *   xq, xk, ga, gb : [B, T, H, dk] dtype      xv, gw : [B, T, H, dv] dtype
 *   conv_q, conv_k : [H*dk, conv_width] fp32  conv_v : [H*dv, conv_width] fp32
 *                    (channel h*d + c)
 *   q, k, alpha, b : [B, T, H, dk] dtype      v, w   : [B, T, H, dv] dtype
 *   cu_seqlens     : NULL, or device int32[num_seqs + 1] with B == 1 (the
 *                    convolution restarts at each sequence)
 *   dtype          : GDN2_BF16 or GDN2_F32;  dk, dv : 64 or 128
 *   H              : H * max(dk, dv) < 2^24 (rows are addressed with 32-bit
 *                    byte offsets), else GDN2_ERR_INVALID_ARG
 * Outputs must not equal an input or each other (GDN2_ERR_INVALID_ARG).
 * The sigmoids and the L2 norm use the hardware reciprocal and reciprocal
 * square root (about 1 ulp each).  The outputs are the inputs of gdn2_fwd.
 */
int gdn2_prologue(const void* xq, const void* xk, const void* xv, const void* ga,
                  const void* gb, const void* gw, const float* conv_q, const float* conv_k,
                  const float* conv_v, int32_t conv_width, float l2_eps, void* q, void* k,
                  void* v, void* alpha, void* b, void* w, const int32_t* cu_seqlens,
                  int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                  int32_t dtype, void* stream);

/*
 * gdn2_epilogue -- the mixer's readout after the recurrence (same passage:
 * an RMSNorm times a SiLU output gate, before the out projection):
 *     y = o / sqrt(mean_c o[c]^2 + eps) * gamma * SiLU(g)
 * per (token, head) over the dv channels, in one pass over HBM.
 *   o, g  : [rows, H, dv] in_dtype (o as gdn2_fwd writes it; g the gate's
 *           pre-activation)
 *   gamma : [dv] fp32 weight shared by the heads, or NULL (= 1)
 *   y     : [rows, H, dv] out_dtype (in_dtype or GDN2_F32); not o or g
 */
int gdn2_epilogue(const void* o, const void* g, const float* gamma, float eps, void* y,
                  int32_t rows, int32_t H, int32_t dv, int32_t in_dtype, int32_t out_dtype,
                  void* stream);

/*
 * gdn2_fwd_noalloc -- gdn2_fwd_gates without a workspace argument, for
 * callers that cannot allocate device memory around the call: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * call itself allocates nothing (no hipMalloc, no allocating library call).
 *
 * Where gdn2_fwd_gates would need a workspace (long sequences with few
 * (sequence, head) pairs, packed batches), it uses a device array of
 * GDN2_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU it runs
 * on, until the process ends.  Its device address is looked up on the first
 * call on a device (with that device current).
 *  - Sizes whose gdn2_fwd_workspace_size(...) exceeds
 *    GDN2_NOALLOC_SCRATCH_BYTES: GDN2_ERR_WORKSPACE, before anything is
 *    launched; except fp32 inputs at dk = 128, whose token-serial forward
 *    then runs unsegmented, with no workspace.  A HIP error in the lookup:
 *    GDN2_ERR_HIP.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents (nothing in it needs to start at zero: each call writes
 *    what it reads).  Calls that overlap on one GPU (other streams, other
 *    host threads) race on it and give undefined results; serialise them.
 * Other arguments, checks and results as for gdn2_fwd_gates (bit-identical
 * outputs for the same inputs).
 */
#define GDN2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int gdn2_fwd_noalloc(const void* q, const void* k, const void* v, const void* alpha,
                     const void* b, const void* w, int32_t gates, int32_t in_dtype,
                     const float* S0, void* o, int32_t out_dtype, float* S_T,
                     const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                     int32_t H, int32_t dk, int32_t dv, void* stream);

/*
 * gdn2_fwd_ex -- gdn2_fwd_gates with a choice of erase reading (gdn2_erase).
 * GDN2_ERASE_READ is gdn2_fwd_gates itself.  GDN2_ERASE_ROWS runs the
 * recurrence token by token in fp32 (any dtype, dk and dv 64 or 128, dense or
 * packed), one wave per (sequence, head, 16 value columns): exact up to fp32
 * rounding, without the chunked algorithm's speed.  Long sequences with few
 * (sequence, head) pairs are split into segments under the same plan (and
 * the same workspace, gdn2_fwd_workspace_size) as gdn2_fwd_gates: a pass
 * composes each segment's affine state map, the maps are chained into the
 * segments' start states, and every segment then runs from its start.
 * erase outside gdn2_erase: GDN2_ERR_INVALID_ARG; workspace missing or too
 * small: GDN2_ERR_WORKSPACE.
 */
int gdn2_fwd_ex(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                const void* w, int32_t gates, int32_t erase, int32_t in_dtype, const float* S0,
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

/*
 * gdn2_decode_ex -- gdn2_decode_gates with a choice of erase reading
 * (gdn2_erase).  Under GDN2_ERASE_ROWS the step is
 *     S' = Diag(alpha) S,  r = S'^T k,  S <- S' + k x^T - (b (.) k) r^T,
 *     o = S'^T q + (q . k) x - (q . (b (.) k)) r,   x = w (.) v,
 * still one read and one write of the state.
 */
int gdn2_decode_ex(const void* q, const void* k, const void* v, const void* alpha,
                   const void* b, const void* w, int32_t gates, int32_t erase, int32_t in_dtype,
                   float* S, void* o, int32_t out_dtype, int32_t N, int32_t H, int32_t dk,
                   int32_t dv, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H */
