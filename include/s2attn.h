/*
 * s2attn.h - C ABI of the MI355X (gfx950) Shifted Sparse Attention library.
 *
 * The operation (AIMech curated page "LongLoRA and Shifted Sparse Attention
 * (S^2-Attn)", opening definition): projected queries, keys and values are
 * split along the head axis into two equal halves; the second half is rolled
 * by -shift along the sequence (the pages use shift = G/2); the sequence is
 * cut into N/G groups of G tokens; causal softmax attention with logit scale
 * 1/sqrt(D) runs inside each group only ("LongLoRA: Efficient 100k Context
 * LLM Fine-Tuning Guide", section "How Shifted Short Attention Works"); the
 * second half's output is rolled back by +shift.  The roll is circular: the
 * last group of a shifted head holds the last `shift` tokens followed by the
 * first `shift` tokens, causal in that rolled order.
 *
 * Tensors (all row-major and contiguous, bfloat16 unless stated otherwise):
 *   q, out, dout, dq : [B, N, H,   D]
 *   k, v, dk, dv     : [B, N, Hkv, D]
 *   lse              : [B, H, N] float32, natural-log log-sum-exp of each
 *                      row's scaled logits, indexed by original position.
 * Heads h >= H/2 are the shifted half.  Grouped-query sharing: q head h reads
 * k/v head h / (H/Hkv), rolled by q head h's shift.
 *
 * Ownership: every pointer is device memory owned by the caller.  The library
 * allocates nothing and keeps no pointer after a call returns.  Outputs must
 * not overlap inputs or each other.  Tensor pointers must be 16-byte aligned.
 * Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 * null stream); results are ready once the stream is synchronised.
 *
 * Errors: every call returns S2ATTN_OK (0) or a negative status and never
 * throws.  Arguments are checked before any GPU work is enqueued, so a call
 * that fails with S2ATTN_EINVAL or S2ATTN_EUNSUPPORTED has no effect.
 * S2ATTN_EHIP reports a HIP launch/runtime error.  Faults during kernel
 * execution surface at stream synchronisation.  s2attn_last_error() gives a
 * human-readable detail of the calling thread's most recent failure.
 * The library holds no global mutable state apart from that per-thread
 * message; concurrent calls on different streams are safe.
 *
 * Accepted shapes: B >= 0, N >= 0, H >= 1, 1 <= Hkv, H % Hkv == 0, G >= 1,
 * N % G == 0, 0 <= shift < G; with shift > 0, H and Hkv must be even (so the
 * shifted q heads read exactly the shifted k/v heads).  D must be 64 or 128
 * (else S2ATTN_EUNSUPPORTED).  64 * H * D must stay below 2^31 (the kernels
 * address 64-row tiles with 32-bit offsets).  B == 0 or N == 0 is a valid
 * empty call.
 */
#ifndef S2ATTN_H
#define S2ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define S2ATTN_OK 0
#define S2ATTN_EINVAL (-1)
#define S2ATTN_EUNSUPPORTED (-2)
#define S2ATTN_EHIP (-3)

/* Which q heads are shifted (s2attn_fwd_ex / s2attn_bwd_ex). */
#define S2ATTN_HEADS_SECOND_HALF 0 /* heads H/2 .. H-1, as every other entry point does */
#define S2ATTN_HEADS_ALTERNATE 1   /* the q heads of the odd k/v heads */

/*
 * Forward pass.  Writes out (and lse unless lse is NULL).
 * Reads q, k, v; the group split and the rolls are folded into index
 * arithmetic, nothing is copied.
 */
int s2attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
               int B, int N, int H, int Hkv, int D, int G, int shift, void* stream);

/*
 * Workspace bytes s2attn_bwd needs: two float32 [B, H, N] row statistics,
 * -Delta[b, h, n] = -sum_d dout * out and -lse[b, h, n] * log2(e), each
 * starting on a 256-byte boundary (8 bytes per (b, h, n) row in all).
 */
size_t s2attn_bwd_workspace_size(int B, int N, int H, int Hkv, int D);

/*
 * Backward pass: gradients of out w.r.t. q, k, v for the upstream gradient
 * dout (the calculus of the forward; the pages do not spell it out).
 * out and lse must be the forward's results for the same q, k, v.
 * dq, dk, dv are overwritten (not accumulated into).  `workspace` is device
 * memory of at least s2attn_bwd_workspace_size() bytes (256-byte aligned),
 * clobbered by the call.  The kernels recompute P from the forward's own
 * logits (q times log2(e)/sqrt(D) rounded to bf16 once, formed as q is
 * loaded), so each row of P sums to one against lse.  Deterministic: no
 * atomics.
 */
int s2attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
               const void* dout, void* dq, void* dk, void* dv,
               int B, int N, int H, int Hkv, int D, int G, int shift,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * s2attn_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation with no workspace argument.  The row statistics live in
 * a device scratch array inside the library, 32 MiB per GPU, held from the
 * first call on that GPU until the process ends; the call rejects
 * (S2ATTN_EINVAL) shapes whose statistics exceed it, i.e. B*H*N above
 * 4,194,304 rows.  It allocates nothing and calls no allocating routine.
 * Every call on one GPU uses that GPU's one scratch array: calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  The scratch used is that of the calling
 * thread's current HIP device, so stream (and every tensor) must belong to
 * that device.  No RoPE; heads H/2 .. H-1 are shifted.
 */
int s2attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       int B, int N, int H, int Hkv, int D, int G, int shift, void* stream);

/*
 * The backward in stages: the same kernels s2attn_bwd enqueues, in the same
 * order, for callers that want to schedule or time them separately.
 *   s2attn_bwd_preprocess  the row statistics (-Delta, -lse*log2(e)) from
 *                          out, dout and the forward's lse, into the
 *                          workspace
 *   s2attn_bwd_dkdv        dk, dv
 *   s2attn_bwd_dq          dq
 * dkdv and dq do not depend on each other and may run on different streams
 * once preprocess has completed; both only read the workspace.  Arguments
 * and the workspace are those of s2attn_bwd (workspace of
 * s2attn_bwd_workspace_size() bytes).
 */
int s2attn_bwd_preprocess(const void* out, const void* dout, const float* lse,
                          int B, int N, int H, int D,
                          void* workspace, size_t workspace_bytes, void* stream);
int s2attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                    void* dk, void* dv,
                    int B, int N, int H, int Hkv, int D, int G, int shift,
                    const void* workspace, size_t workspace_bytes, void* stream);
int s2attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq,
                  int B, int N, int H, int Hkv, int D, int G, int shift,
                  const void* workspace, size_t workspace_bytes, void* stream);

/*
 * RoPE with linear position interpolation, fused ahead of the attention
 * ("LoRA for Long-Context Adaptation", sections "Why vanilla LoRA
 * under-delivers on long context" and "Position interpolation"): before the
 * roll, each adjacent pair (x[2i], x[2i+1]) of q and k at original position p
 * is rotated counter-clockwise by (p / pos_scale) * rope_base^(-2i/D).
 * q and k are passed unrotated; lse refers to the rotated logits.
 * rope_base > 0 and pos_scale > 0 must be finite.
 *
 * s2attn_fwd_rope needs a workspace for the rotated k ([B, N, Hkv, D] bf16);
 * q is rotated inside the attention kernel.  k is rotated once per call by a
 * pass of its own (each k row is staged by every q tile of its group, so
 * rotating it inside the attention kernel would repeat the rotation up to
 * G/256 times); on one MI355X at B 1, N 32768, Hkv 8, D 128 that pass takes
 * about 22 us (67 MB read and written), under 1% of the forward call.
 */
size_t s2attn_fwd_rope_workspace_size(int B, int N, int H, int Hkv, int D);
int s2attn_fwd_rope(const void* q, const void* k, const void* v, void* out, float* lse,
                    int B, int N, int H, int Hkv, int D, int G, int shift,
                    double rope_base, double pos_scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of s2attn_fwd_rope: dq and dk are gradients w.r.t. the unrotated
 * q and k (passed back through the transposed rotation).  The workspace holds
 * the two row statistics, bf16(rotated q * log2(e)/sqrt(D)) and bf16(rotated
 * k): q and k are rotated once per call by a pass of their own (every q row
 * is re-read by each k/v tile of its group, every k row by each q tile, so
 * rotating them inside those kernels would repeat the rotation G/128 and
 * G/256 times over).  On one MI355X at B 1, N 32768, H 64, Hkv 8, D 128 the
 * two passes take about 0.19 ms (q 537 MB, k 67 MB), under 2% of the
 * backward call.
 */
size_t s2attn_bwd_rope_workspace_size(int B, int N, int H, int Hkv, int D);
int s2attn_bwd_rope(const void* q, const void* k, const void* v, const void* out,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    int B, int N, int H, int Hkv, int D, int G, int shift,
                    double rope_base, double pos_scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The general entry points: every option of the calls above, plus the choice
 * of shifted heads.
 *   head_pattern  S2ATTN_HEADS_SECOND_HALF: heads H/2 .. H-1 are shifted
 *                 ("LongLoRA and Shifted Sparse Attention (S^2-Attn)",
 *                 opening definition; needs even H and Hkv when shift > 0).
 *                 S2ATTN_HEADS_ALTERNATE: alternate heads are shifted ("LoRA
 *                 for Long-Context Adaptation", section "Shifted sparse
 *                 attention": heads 1, 3, 5, ...).  With grouped-query
 *                 sharing this reads as the q heads of the odd k/v heads, so
 *                 each k/v head's rows are rolled one way; without sharing it
 *                 is exactly the odd heads.
 *   rope_base     0 for no RoPE; otherwise RoPE with position interpolation
 *                 as in s2attn_fwd_rope (rope_base > 0, pos_scale > 0, finite).
 * Workspaces: the forward needs s2attn_fwd_rope_workspace_size() bytes when
 * RoPE is on and none otherwise (workspace may be NULL); the backward needs
 * s2attn_bwd_rope_workspace_size() or s2attn_bwd_workspace_size() bytes.
 * Everything else (layouts, ownership, errors) is as for s2attn_fwd and
 * s2attn_bwd; the backward must be given the forward's head_pattern and RoPE.
 */
int s2attn_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                  int B, int N, int H, int Hkv, int D, int G, int shift,
                  int head_pattern, double rope_base, double pos_scale,
                  void* workspace, size_t workspace_bytes, void* stream);
int s2attn_bwd_ex(const void* q, const void* k, const void* v, const void* out,
                  const float* lse, const void* dout, void* dq, void* dk, void* dv,
                  int B, int N, int H, int Hkv, int D, int G, int shift,
                  int head_pattern, double rope_base, double pos_scale,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * LoRA-adapted q/k/v projections, the step ahead of the attention ("LoRA for
 * Long-Context Adaptation", section "Why vanilla LoRA under-delivers on long
 * context": two small trained matrices A (d x r) and B (r x d) added to each
 * frozen target projection; "Practical recipe": the attention projections
 * are the targets).  The formula itself is lost from the page; the reading
 * implemented is, for each target p in (q, k, v) and token rows x,
 *     y_p = x W_p + scale * (x A_p) B_p.
 *
 * Layouts (bf16, row-major, contiguous, 16-byte aligned):
 *   x            [M, d_in]          token rows (M = B * N)
 *   wq_t         [width_q, d_in]    W_q transposed: one row per output column
 *   wk_t, wv_t   [width_kv, d_in]
 *   aq_t ...     [r, d_in]          A_p transposed
 *   bq_t         [width_q, r]       B_p transposed; bk_t, bv_t [width_kv, r]
 *   q            [M, width_q]       = [B, N, H, D] with width_q = H * D
 *   k, v         [M, width_kv]      = [B, N, Hkv, D] with width_kv = Hkv * D
 * This is the weight[out][in] orientation of a linear layer.
 *
 * Limits: d_in, width_q and width_kv multiples of 64 (>= 64, d_in <= 2^20);
 * r = 0 (no adapter: plain projections; the A, B pointers and the
 * workspace may then be NULL) or a multiple of 8 up to 1024; scale finite.
 * The workspace (s2attn_lora_qkv_workspace_size() bytes, 256-byte aligned)
 * holds, after the call, scale * x A_p for the three targets side by side
 * ([M, 3r] bf16): the low-rank activations a backward pass needs.  Products
 * accumulate in float32; that intermediate and the outputs are rounded to
 * bf16 once.  Outputs must not overlap any input or each other.
 */
size_t s2attn_lora_qkv_workspace_size(int M, int r);
int s2attn_lora_qkv_fwd(const void* x, int M, int d_in,
                        const void* wq_t, const void* wk_t, const void* wv_t,
                        int width_q, int width_kv,
                        const void* aq_t, const void* ak_t, const void* av_t,
                        const void* bq_t, const void* bk_t, const void* bv_t,
                        int r, double scale,
                        void* q, void* k, void* v,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of s2attn_lora_qkv_fwd (the calculus of its forward; the pages do
 * not spell it out).  The pretrained W_p are frozen, so the call returns the
 * input gradient and the adapters' gradients for upstream gradients dq, dk,
 * dv ([M, width_q], [M, width_kv], [M, width_kv] bf16):
 *   dx   = sum_p dy_p W_p^T + scale * (dy_p B_p^T) A_p^T     [M, d_in]
 *   dA_p = scale * x^T (dy_p B_p^T)      written transposed, [r, d_in]
 *   dB_p = (scale * x A_p)^T dy_p        written transposed, [width_p, r]
 * `t` is the forward's low-rank activations (the first M * 3r bf16 of the
 * forward's workspace after the call); dB is formed from it, so it carries
 * the forward's bf16 rounding.  Weights, layouts and limits are those of
 * s2attn_lora_qkv_fwd; outputs are overwritten.  With r = 0 only dx is
 * computed and the adapter pointers, t and the workspace may be NULL.  The
 * workspace (s2attn_lora_qkv_bwd_workspace_size() bytes, 256-byte aligned,
 * clobbered) holds scale * dy_p B_p^T and the fixed-order partial sums of the
 * token reductions; the result is deterministic.
 */
size_t s2attn_lora_qkv_bwd_workspace_size(int M, int d_in, int width_q, int width_kv, int r);
int s2attn_lora_qkv_bwd(const void* x, int M, int d_in,
                        const void* wq_t, const void* wk_t, const void* wv_t,
                        int width_q, int width_kv,
                        const void* aq_t, const void* ak_t, const void* av_t,
                        const void* bq_t, const void* bk_t, const void* bv_t,
                        int r, double scale, const void* t,
                        const void* dq, const void* dk, const void* dv,
                        void* dx, void* daq_t, void* dak_t, void* dav_t,
                        void* dbq_t, void* dbk_t, void* dbv_t,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* s2attn_strerror(int status);

/* Detail of the calling thread's most recent failed call ("" if none). */
const char* s2attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* S2ATTN_H */
