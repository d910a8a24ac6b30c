/*
 * lightning_la.h -- C ABI of the MI355X (gfx950) causal linear-attention
 * ("Lightning Attention") layer: chunked prefill and single-token decode.
 *
 * The layer (per batch element b and head h, tokens t at absolute positions
 * pos0 + t):
 *   qh_t = RoPE(RMSNorm(q_t)), kh_t = RoPE(RMSNorm(k_t))     (v is not normalized)
 *   S_t  = S_{t-1} + kh_t v_t^T                               (fp32 state, D x D)
 *   o_t  = sigmoid(g_t) * (qh_t S_t)                          (elementwise gate)
 *
 * Sources (pages cited by title and section):
 *   - State update S_t = S_{t-1} + k_t v_t^T: "MiniCPM-SALA: Hybridizing Sparse and
 *     Linear Attention for Efficient Long-Context Modeling" (paper digest),
 *     前置知识 > 线性注意力 (Linear Attention).
 *   - QK-normalization, MHA heads (GQA converted to MHA), output gating on the
 *     linear layers: "創新Transformer！面壁基於稀疏-線性混合架構SALA訓練9B模型"
 *     (MiniCPM-SALA technical-report rendering), 04 技術報告 > 02 模型架構 >
 *     (3) 線性注意力模塊; also "9B端側開源模型跑通百萬上下文，面壁全新稀疏-線性混合
 *     注意力" (QbitAI article), architecture section.
 *   - RoPE kept on the linear layers (HyPE): technical-report rendering,
 *     02 模型架構 > (4) 混合位置編碼.
 * Readings where the pages are silent: the readout o_t = q_t S_t sees token t
 * itself; no decay, feature map, normalizing denominator or 1/sqrt(D) scale;
 * RMSNorm n_i = w_i x_i / sqrt(mean(x^2) + eps) over the head dimension;
 * rotate-half RoPE pairing (i, i + D/2) with theta_i = rope_base^(-2i/D) applied
 * after the norm; the gate is sigmoid of per-element logits of o's shape and
 * never touches S.
 *
 * Layouts (row-major, no padding):
 *   q, k, v, gate logits, o : bf16 [B, T, H, D]   (decode: [B, H, D])
 *   S_in, S_out, S          : fp32 [B, H, D, D], S[i][j] = sum_t kh_t[i] v_t[j]
 *   q_norm_w, k_norm_w      : fp32 [D], or NULL for all-ones weights
 * Supported: D == 128, B, H >= 1, T >= 1, chunk in {0 (= default = 64), 64, 128,
 * 256}, rope_base finite and > 0, rms_eps finite and >= 0.
 *
 * Ownership and asynchrony: every pointer (except where noted) is a device
 * pointer owned by the caller.  The library allocates no memory and keeps no
 * mutable global state (except la_prefill_noalloc's static scratch, below);
 * calls are re-entrant.  A call validates its arguments,
 * enqueues its kernels on `stream` (a hipStream_t passed as void*; NULL = the
 * null stream) and returns; results are valid once the caller synchronizes
 * that stream.
 *
 * Errors: all validation happens before anything is enqueued; on any status
 * other than LA_OK nothing was launched and no output was touched (except
 * LA_ERR_HIP, returned when a launch itself fails; device faults surface at
 * the caller's synchronization).  No C++ exception crosses this interface.
 * Graph capture: every entry point except la_prefill_varlen only enqueues
 * kernels and can be captured into a HIP graph; la_prefill_varlen refuses a
 * capturing stream with LA_ERR_CAPTURING.
 */
#ifndef LIGHTNING_LA_H
#define LIGHTNING_LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LA_OK = 0,
  LA_ERR_NULL_PTR = 1,    /* a required pointer is NULL                              */
  LA_ERR_BAD_SHAPE = 2,   /* B, T or H < 1, or a size product overflows               */
  LA_ERR_UNSUPPORTED = 3, /* D != 128, chunk not in {0, 64, 128, 256}, or a bad
                             rope_base / rms_eps                                     */
  LA_ERR_ALIGNMENT = 4,   /* a pointer is not 16-byte aligned                          */
  LA_ERR_ALIASING = 5,    /* o overlaps an input, or S_out overlaps an activation      */
  LA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than la_prefill_workspace_bytes */
  LA_ERR_HIP = 7,         /* a kernel launch failed                                    */
  LA_ERR_CAPTURING = 8    /* la_prefill_varlen on a stream that is capturing a graph   */
} la_status;

typedef uint16_t la_bf16; /* raw bfloat16 bits */

/* Version of this interface (major * 10000 + minor * 100 + patch). */
int la_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* la_status_string(la_status s);

/*
 * Bytes of device workspace la_prefill needs for this shape and chunk (0 for an
 * invalid shape).  A segment is a run of consecutive chunks handled by one
 * workgroup.  When the B * H sequence-heads alone fill the GPU (at least 256 of
 * them, and the last round of 256 workgroups at least a quarter used) or the
 * input is one chunk long, each (b, h) is one segment: one kernel reads k and v
 * once, starts from S_in and writes S_out, and the workspace is a token 256
 * bytes.  Otherwise the workspace holds one fp32 D x D state per (b, h,
 * segment): a first kernel sums each segment's Kh^T V, a scan forms the prefix
 * states, and the output kernel walks each segment from its prefix.
 */
size_t la_prefill_workspace_bytes(int B, int T, int H, int D, int chunk);

/*
 * Chunked prefill over T tokens starting at absolute position pos0.
 *   q, k, v, gate_logits : [B, T, H, D] bf16 inputs.
 *   S_in  : [B, H, D, D] fp32 initial state, or NULL for zeros.  May equal S_out
 *           (in-place carry between segments of a long sequence).
 *   S_out : [B, H, D, D] fp32 final state (the state after token T - 1).
 *   o     : [B, T, H, D] bf16 gated output; must not overlap any input.
 *   chunk : tokens per chunk of the chunked evaluation: 0 (= 64), 64, 128 or 256.
 *           The result is the same closed form for every chunk; the chunk only
 *           decides which token pairs go through the bf16 score products and
 *           which through the bf16 state operand.  64 is the fast path; 128
 *           and 256 run a single-buffered kernel that stages k and v of a
 *           chunk's earlier 64-row blocks again for every later block.
 *   rope_base : RoPE base (10000 in the workloads); rms_eps : RMSNorm epsilon.
 *   workspace : device buffer of at least la_prefill_workspace_bytes(...) bytes;
 *               its contents on entry are irrelevant and are clobbered.
 * Arithmetic: bf16 MFMA products with fp32 accumulation; fp32 state; RMSNorm,
 * RoPE and gate in fp32 with RoPE angles reduced in double precision.
 */
la_status la_prefill(const la_bf16* q, const la_bf16* k, const la_bf16* v,
                     const la_bf16* gate_logits, const float* S_in, float* S_out, la_bf16* o,
                     int B, int T, int H, int D, int64_t pos0, int chunk, float rope_base,
                     float rms_eps, const float* q_norm_w, const float* k_norm_w,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * la_prefill that also records caller-created HIP events (hipEvent_t passed as
 * void*) on `stream` at its kernel boundaries, for per-kernel timing:
 *   events[0] before the chunk-state kernel, events[1] before the state scan,
 *   events[2] before the output kernel, events[3] after the output kernel
 *   (with one segment per (b, h) there is no state kernel or scan: events 0, 1
 *   and 2 all mark the start of the output kernel).
 * n_events must be 4 and every event non-NULL (else LA_ERR_NULL_PTR); the
 * results are identical to la_prefill's.
 */
la_status la_prefill_profiled(const la_bf16* q, const la_bf16* k, const la_bf16* v,
                              const la_bf16* gate_logits, const float* S_in, float* S_out,
                              la_bf16* o, int B, int T, int H, int D, int64_t pos0, int chunk,
                              float rope_base, float rms_eps, const float* q_norm_w,
                              const float* k_norm_w, void* workspace, size_t workspace_bytes,
                              void* stream, void* const* events, int n_events);

/*
 * la_prefill without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops that must not call
 * hipMalloc, harnesses that forbid allocation.  Same arguments, results and
 * errors as la_prefill otherwise.
 * The segment states live in a static device array of the library ("scratch",
 * 64 MiB = 1024 fp32 128 x 128 states; each GPU the library runs on holds its own
 * copy from the first call on it until the process ends).  The call allocates
 * nothing: the first call on a device looks up the array's device address
 * (hipGetSymbolAddress) and keeps it.  When la_prefill's plan would need more
 * than 1024 segment states, the call cuts each (b, h) into fewer, longer
 * segments, down to one segment per (b, h), which keeps no states at all (same
 * closed form; the fp32 state sums are grouped differently, so results may
 * differ from la_prefill's by rounding).  Every shape la_prefill accepts is
 * served.
 * Every call on a GPU shares that GPU's scratch: calls that overlap in time on
 * one GPU (on different streams, or from several threads without ordering)
 * race and must not be issued; calls ordered on one stream are safe.  The
 * scratch needs no clearing: each call writes every state it reads.
 */
la_status la_prefill_noalloc(const la_bf16* q, const la_bf16* k, const la_bf16* v,
                             const la_bf16* gate_logits, const float* S_in, float* S_out, la_bf16* o,
                             int B, int T, int H, int D, int64_t pos0, int chunk, float rope_base,
                             float rms_eps, const float* q_norm_w, const float* k_norm_w, void* stream);

/*
 * Variable-length batch ("varlen"): nseq sequences packed along the token axis,
 * for ragged prefill batches and for mixed batches of prefill chunks and decode
 * steps.  Sequence b owns packed tokens [cu_seqlens[b], cu_seqlens[b + 1]) of
 * q, k, v, gate_logits and o ([total_T, H, D] bf16), starts at absolute
 * position pos0[b] and carries its own state S_in[b] -> S_out[b] ([nseq, H, D, D]
 * fp32).  Each sequence gets what la_prefill (or, for one token, la_decode_step)
 * gives it alone; the length mix only changes how the work is cut up.  The pages
 * time prefill (time to first token) and prefill plus decode ("創新Transformer！
 * 面壁基於稀疏-線性混合架構SALA訓練9B模型，端側跑通百萬上下文", 05 計算效率測試) and
 * name batching and concurrent requests as unstudied ("MiniCPM-SALA: Hybridizing
 * Sparse and Linear Attention for Efficient Long-Context Modeling", 独立分析的弱点);
 * this entry point is the batched form of the same layer.
 *   cu_seqlens : HOST int32 [nseq + 1]: cu_seqlens[0] = 0, nondecreasing,
 *                cu_seqlens[nseq] = total_T.  A sequence may be empty (its
 *                S_out[b] = S_in[b]) or a single token (a decode step: the
 *                decode kernel serves it).
 *   pos0       : HOST int64 [nseq], or NULL for all zeros.
 *   q, k, v, gate_logits, o may be NULL when total_T == 0.
 *   S_in       : device [nseq, H, D, D] or NULL (zeros); may equal S_out.
 *   chunk, rope_base, rms_eps, q_norm_w, k_norm_w : as for la_prefill.
 *   workspace  : at least la_prefill_varlen_workspace_bytes(...) bytes.
 * The call builds its work tables on the host and copies them into the front
 * of the workspace with hipMemcpyAsync on `stream` before the kernels, so it
 * returns once that (pageable) copy has been staged.  Errors as for la_prefill;
 * LA_ERR_BAD_SHAPE also covers malformed cu_seqlens.
 * Graph capture: the table copy reads host memory that lives only for the
 * call, so the call cannot be captured into a HIP graph.  On a stream that is
 * capturing (hipStreamIsCapturing) it returns LA_ERR_CAPTURING after the other
 * checks and enqueues nothing.  Every other entry point only enqueues kernels
 * (and reads no host memory at run time), so those can be captured.
 */
size_t la_prefill_varlen_workspace_bytes(int nseq, const int32_t* cu_seqlens, int H, int D, int chunk);

la_status la_prefill_varlen(const la_bf16* q, const la_bf16* k, const la_bf16* v,
                            const la_bf16* gate_logits, const int32_t* cu_seqlens, const int64_t* pos0,
                            const float* S_in, float* S_out, la_bf16* o, int nseq, int total_T, int H,
                            int D, int chunk, float rope_base, float rms_eps, const float* q_norm_w,
                            const float* k_norm_w, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dense projection y = x W^T (the nn.Linear layout: W is [N, K]), bf16 inputs,
 * fp32 accumulation, bf16 output; the q/k/v/gate and output projections around
 * the layer in "創新Transformer！面壁基於稀疏-線性混合架構SALA訓練9B模型，端側跑通百萬上下文"
 * (04 技術報告 > 02 模型架構 > (3) 線性注意力模塊: hidden 4096, 32 heads of 128).
 *   x : [M, K], w : [N, K], y : [M, N], all row-major device buffers; y must not
 *       overlap x or w.
 * Supported: K % 64 == 0, N % 256 == 0, M >= 1 (LA_ERR_UNSUPPORTED otherwise).
 */
la_status la_linear(const la_bf16* x, const la_bf16* w, la_bf16* y, int64_t M, int N, int K, void* stream);

/*
 * Bytes of workspace la_layer_forward needs: q, k, v, gate and o buffers of
 * B * T * H * D bf16 each (rounded to 256 bytes) plus la_prefill's workspace.
 */
size_t la_layer_workspace_bytes(int B, int T, int H, int D, int chunk);

/*
 * One linear-attention layer forward: [q | k | v | g] = x W_qkvg^T (one
 * projection whose four column blocks land in four [B, T, H, D] buffers of the
 * workspace), then la_prefill on them, then y = o W_o^T.
 *   x        : [B, T, hidden] bf16
 *   w_qkvg   : [4 H D, hidden] bf16, rows ordered q heads, k heads, v heads, gate
 *   w_o      : [hidden, H D] bf16
 *   S_in, S_out, pos0, chunk, rope_base, rms_eps, q_norm_w, k_norm_w : as la_prefill
 *   y        : [B, T, hidden] bf16; must not overlap x, the weights or the states
 * Supported: D == 128, hidden % 256 == 0, (H D) % 256 == 0.
 */
la_status la_layer_forward(const la_bf16* x, const la_bf16* w_qkvg, const la_bf16* w_o, const float* S_in,
                           float* S_out, la_bf16* y, int B, int T, int hidden, int H, int D, int64_t pos0,
                           int chunk, float rope_base, float rms_eps, const float* q_norm_w,
                           const float* k_norm_w, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace la_backward needs (0 for an invalid shape or a chunk other
 * than 0 / 64): two sets of segment states, bf16 gradients of the rotated q and
 * k ([B, T, H, D] each) and 2 MiB for the norm-weight gradient parts.
 */
size_t la_backward_workspace_bytes(int B, int T, int H, int D, int chunk);

/*
 * Gradients of la_prefill for a loss with gradient d_o of o ([B, T, H, D] bf16)
 * and dS_out of S_out ([B, H, D, D] fp32, or NULL for zeros): the reverse mode of
 * the recurrence S_t = S_{t-1} + k_t v_t^T, o_t = sigmoid(g_t) * (q_t S_t) of
 * "MiniCPM-SALA: Hybridizing Sparse and Linear Attention for Efficient
 * Long-Context Modeling" (前置知识 > 线性注意力), through the output gate, RoPE and
 * QK-RMSNorm of the report's linear-attention module.  The pages train the
 * converted linear layers ("創新Transformer！面壁基於稀疏-線性混合架構SALA訓練9B模型，
 * 端側跑通百萬上下文", 04 技術報告 > 03 模型訓練).
 *   q, k, v, gate_logits, S_in, pos0, rope_base, rms_eps, q_norm_w, k_norm_w :
 *       the forward call's arguments (S_in may be NULL)
 *   dq, dk, dv, dgate : [B, T, H, D] bf16 outputs
 *   dS_in             : [B, H, D, D] fp32 output (gradient of the initial state)
 *   dq_norm_w, dk_norm_w : [D] fp32 outputs or NULL; without norm weights they are
 *       the gradients at weights of one
 *   chunk : 0 or 64
 * Outputs must not overlap each other, the inputs or the workspace.  The
 * forward is recomputed inside the call (segment states and the pre-gate output).
 */
la_status la_backward(const la_bf16* q, const la_bf16* k, const la_bf16* v, const la_bf16* gate_logits,
                      const float* S_in, const la_bf16* d_o, const float* dS_out, la_bf16* dq, la_bf16* dk,
                      la_bf16* dv, la_bf16* dgate, float* dS_in, float* dq_norm_w, float* dk_norm_w, int B,
                      int T, int H, int D, int64_t pos0, int chunk, float rope_base, float rms_eps,
                      const float* q_norm_w, const float* k_norm_w, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * la_backward with the forward's segment states taken from the workspace of the
 * la_prefill call that computed the same forward (same q, k, v, gate_logits,
 * S_in, B, T, H, D, pos0, chunk, rope_base, rms_eps and norm weights, its
 * workspace not written since; la_prefill_varlen and la_prefill_noalloc
 * workspaces do not qualify).  That call's state pass and scan already formed the
 * state at every segment start, so the backward's own forward state pass (a read
 * of k and v) and scan are skipped; the results are those of la_backward, bit for
 * bit.  The reverse mode is that of la_backward ("MiniCPM-SALA: Hybridizing
 * Sparse and Linear Attention for Efficient Long-Context Modeling", 前置知识 >
 * 线性注意力; the report's 04 技術報告 > 03 模型訓練).
 *   fwd_workspace : that call's workspace (read only; NULL: recompute, as
 *       la_backward), fwd_workspace_bytes its size.  When la_prefill walks each
 *       (b, h) in one workgroup for this shape it keeps no states, and they are
 *       recomputed.
 * Other arguments as la_backward.  Errors as la_backward, plus LA_ERR_WORKSPACE
 * when fwd_workspace_bytes is below la_prefill_workspace_bytes for the shape, and
 * LA_ERR_ALIASING when an output or the workspace overlaps fwd_workspace.
 */
la_status la_backward_saved(const la_bf16* q, const la_bf16* k, const la_bf16* v, const la_bf16* gate_logits,
                            const float* S_in, const la_bf16* d_o, const float* dS_out, la_bf16* dq, la_bf16* dk,
                            la_bf16* dv, la_bf16* dgate, float* dS_in, float* dq_norm_w, float* dk_norm_w, int B,
                            int T, int H, int D, int64_t pos0, int chunk, float rope_base, float rms_eps,
                            const float* q_norm_w, const float* k_norm_w, void* workspace, size_t workspace_bytes,
                            const void* fwd_workspace, size_t fwd_workspace_bytes, void* stream);

/*
 * One decode step: one token per sequence at absolute position pos.
 *   q, k, v, gate_logits : [B, H, D] bf16.
 *   S : [B, H, D, D] fp32 state, updated in place (S += kh v^T).
 *   o : [B, H, D] bf16 gated output, o = sigmoid(g) * (qh S_new).
 * Arithmetic: fp32 throughout (no rounding of qh, kh or S to bf16).
 */
la_status la_decode_step(const la_bf16* q, const la_bf16* k, const la_bf16* v,
                         const la_bf16* gate_logits, float* S, la_bf16* o, int B, int H, int D,
                         int64_t pos, float rope_base, float rms_eps, const float* q_norm_w,
                         const float* k_norm_w, void* stream);

/* ---------------------------------------------------------------------------
 * The sparse attention layers of the same hybrid (InfLLM-v2 block selection, no
 * position encoding, output gate): "創新Transformer！面壁基於稀疏-線性混合架構SALA訓練9B
 * 模型，端側跑通百萬上下文", 04 技術報告 > 02 模型架構 > (2) 稀疏注意力模塊 (each query
 * reaches only a few key/value blocks chosen by block selection; dense at ordinary
 * lengths; output gate) and (4) 混合位置編碼 (NoPE in these layers).
 * Readings where the pages are silent: causal softmax attention with scale
 * 1/sqrt(D); blocks of 64 tokens; key block j is scored by its mean key kbar_j and a
 * block of queries by its mean query (a decode step: the query itself):
 * s = qbar . kbar_j over the complete blocks j before the query's block; the topk
 * best (ties to the lower block) plus the query's own block up to the query are
 * attended; o = sigmoid(g) * (attention output).  With at most topk earlier blocks
 * the layer is dense causal attention.
 * Layouts: q, k, v, gate logits, o: bf16 [B, T, H, D] (decode q, gate, o: [B, H, D];
 * caches [B, Tmax, H, D]); block means fp32 [B, H, T / 64, D].
 * Supported: D == 128, block in {0 (= 64), 64}, 1 <= topk <= 64, at most 8192 key
 * blocks per sequence (T or Tmax <= 524288), B and H <= 65535.
 */

/* Workspace of la_sparse_prefill: the key-block means, fp32 [B, H, T / 64, D],
 * then (at the next 256-byte boundary) room for the block choice, int32
 * [B, H, ceil(T / 64), topk], used when sel is NULL (0 for an unsupported shape). */
size_t la_sparse_prefill_workspace_bytes(int B, int T, int H, int D, int block, int topk);

/*
 * Sparse layer over whole sequences from position 0.
 *   q, k, v, gate_logits : [B, T, H, D] bf16;  o : [B, T, H, D] bf16 output.
 *   sel : NULL, or int32 [B, H, ceil(T / 64), topk] output: each query block's chosen
 *         key blocks in increasing order, then -1.
 * Outputs must not overlap the inputs, each other or the workspace.
 */
la_status la_sparse_prefill(const la_bf16* q, const la_bf16* k, const la_bf16* v, const la_bf16* gate_logits,
                            la_bf16* o, int32_t* sel, int B, int T, int H, int D, int block, int topk,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Means of key blocks [first_block, first_block + nblocks) of a key cache
 * k_cache ([B, Tmax, H, D] bf16) into means ([B, H, Tmax / 64, D] fp32), for
 * la_sparse_decode.  A serving loop calls it once per completed block; the blocks
 * named must be filled ((first_block + nblocks) * 64 <= Tmax).
 */
la_status la_sparse_block_means(const la_bf16* k_cache, float* means, int B, int Tmax, int H, int D, int block,
                                int first_block, int nblocks, void* stream);

/*
 * One decode step of the sparse layer per sequence.
 *   q, gate_logits : [B, H, D] bf16, the query of each sequence's newest token,
 *       whose k and v are already in the caches;
 *   k_cache, v_cache : [B, Tmax, H, D] bf16;  means : their block means
 *       (la_sparse_block_means) for every complete block before the newest token's;
 *   lens : device int32 [B], valid tokens per sequence (the newest included), read
 *       on the device; values outside [1, Tmax] are clamped into it;
 *   o : [B, H, D] bf16 output;  sel : NULL or int32 [B, H, topk] output.
 */
la_status la_sparse_decode(const la_bf16* q, const la_bf16* k_cache, const la_bf16* v_cache, const float* means,
                           const la_bf16* gate_logits, const int32_t* lens, la_bf16* o, int32_t* sel, int B,
                           int Tmax, int H, int D, int block, int topk, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_LA_H */
