/*
 * mi355_attn.h - C ABI of the MI355X (gfx950) fused exact-softmax attention
 * forward and backward library, libmi355_attn.so.
 *
 * The operation and its decomposition follow the FlashAttention backward
 * examples of the TileLang pull request "[Example] Introduce split+sum
 * template, and optimize atomic_add performance for bwd examples"
 * (tile-ai/tilelang #940): a forward kernel, a backward preprocess, a
 * backward kernel whose dQ is accumulated either with fp32 atomic adds or
 * through a split-then-sum scheme (the `use_atomic` switch of its sequence
 * diagram), and a backward postprocess.
 *
 * Definitions (per batch b and query head h, with kv = h / groups):
 *   S = scale * Q_h K_kv^T,  S_ij = -inf for j > i when causal,
 *   P = softmax(S) row-wise,  O_h = P V_kv,  LSE_i = ln sum_j exp(S_ij),
 *   Delta_i = sum_d dO_id O_id,  dS = P o (dP - Delta), dP = dO V_kv^T,
 *   dV_kv = sum_h P^T dO_h,  dK_kv = scale * sum_h dS^T Q_h,
 *   dQ_h = scale * dS K_kv.
 *
 * Conventions shared by every call
 *   - Tensors are dense row-major device buffers.  Q, O, dO, dQ are
 *     [batch, seqlen, heads_q, head_dim] (BSHD); K, V, dK, dV are
 *     [batch, seqlen, heads_q/groups, head_dim]; LSE and Delta are
 *     [batch, heads_q, seqlen] fp32.  bf16 tensors hold raw bf16 bit patterns
 *     (uint16_t).  dq_accum, the fp32 dQ accumulator handed from attn_bwd to
 *     attn_bwd_postprocess, is head-major: [batch, heads_q, seqlen, head_dim].
 *   - Every pointer is device memory allocated and owned by the caller; it
 *     must be 16-byte aligned.  The library allocates nothing, frees
 *     nothing, never synchronises and keeps no pointer after a call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream);
 *     the caller keeps every buffer alive until the stream has completed it.
 *   - Return value: ATTN_OK (0) or a negative ATTN_ERR_* code.  All argument
 *     checks run on the host before anything is enqueued, so a call that
 *     fails a check has launched nothing.  ATTN_ERR_HIP reports a launch
 *     failure seen through hipGetLastError after enqueueing.
 */
#ifndef MI355_ATTN_H
#define MI355_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct attn_shape {
  int32_t batch;    /* B >= 1 */
  int32_t seqlen;   /* S >= 1; queries and keys have the same length */
  int32_t heads_q;  /* Hq >= 1 query heads */
  int32_t groups;   /* g >= 1 query heads per KV head; Hq % g == 0, Hkv = Hq / g */
  int32_t head_dim; /* D, 64 or 128 */
} attn_shape;

enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL_PTR = -1,  /* a required pointer is NULL */
  ATTN_ERR_BAD_SHAPE = -2, /* a size out of range, or heads_q not a multiple of groups */
  ATTN_ERR_HEAD_DIM = -3,  /* head_dim not 64 or 128 */
  ATTN_ERR_ALIGN = -4,     /* a tensor base is not 16-byte aligned */
  ATTN_ERR_RANGE = -5,     /* a tensor has >= 2^31 elements, heads_q * head_dim > 2^22,
                              or softmax_scale is not finite and > 0 */
  ATTN_ERR_WORKSPACE = -6, /* workspace NULL or smaller than attn_bwd_workspace_bytes() */
  ATTN_ERR_HIP = -7,       /* the HIP runtime reported a launch error */
  ATTN_ERR_FLAG = -8,      /* causal or use_atomic is not 0 or 1 */
  ATTN_ERR_SCRATCH = -9    /* attn_bwd_noalloc: the problem needs more than its scratch array */
};

/* Static message for a status code (never NULL). */
const char* attn_strerror(int status);

/*
 * Forward: O = softmax(scale * Q K^T [causal]) V and the per-row LSE.
 * (TileLang #940, sequence diagram: attention(Q, K, V, causal, groups, ...)
 * runs flashattn_fwd, which returns O; its backward needs the row
 * normaliser, exported here as LSE.)
 *   q [B,S,Hq,D] bf16, k/v [B,S,Hkv,D] bf16 (inputs)
 *   o [B,S,Hq,D] bf16, lse [B,Hq,S] fp32 natural-log, scale included (outputs)
 *   softmax_scale: finite, > 0 (usually 1/sqrt(D)); causal: 0 or 1.
 * Every element of o and lse is written.
 */
int attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
             attn_shape shape, float softmax_scale, int causal, void* stream);

/*
 * Backward preprocess: Delta_i = sum_d dO_id * O_id in fp32 (the
 * flashattn_bwd_preprocess step of the TileLang #940 examples).
 *   o, dout [B,S,Hq,D] bf16 (inputs); delta [B,Hq,S] fp32 (output).
 *   dq_accum: NULL, or an fp32 [B,Hq,S,D] buffer that is set to zero here,
 *   as the fp32 atomic dQ accumulator of attn_bwd(use_atomic=1) requires.
 */
int attn_bwd_preprocess(const uint16_t* o, const uint16_t* dout, float* delta, float* dq_accum,
                        attn_shape shape, void* stream);

/*
 * Bytes of device workspace attn_bwd and attn_bwd_postprocess need for this
 * problem (0 when none is needed).  Layout, for reference only:
 *   groups > 1: fp32 dK and dV partials, [B,S,Hkv,P,D] each, partial p
 *     the sum over query heads kv*groups + p*groups/P .. of the next
 *     groups/P (one backward workgroup sweeps those heads one after the
 *     other).  P is the smallest divisor of groups with
 *     B * Hkv * P * n_kv_blocks >= 512 (two workgroups per CU of the
 *     256), else groups; n_kv_blocks as below;
 *   use_atomic == 0: fp32 per-KV-block dQ partials, [n_kv_blocks,B,Hq,S,D],
 *     n_kv_blocks = ceil(S / bn), bn = 256 for head_dim 128 and 512 for
 *     head_dim 64 (the backward kernel's key-block height).
 * Returns 0 for an invalid shape.
 */
size_t attn_bwd_workspace_bytes(attn_shape shape, int causal, int use_atomic);

/*
 * Backward: dQ, dK, dV from Q, K, V, dO and the forward's LSE plus the
 * preprocess's Delta (the flashattn_bwd_atomic_add / flashattn_bwd_split
 * pair of the TileLang #940 examples, chosen by use_atomic as its
 * sequence diagram does).
 *   use_atomic = 1: dQ (scaled, fp32) is added with fp32 atomics into
 *     dq_accum, which must hold zeros on entry (attn_bwd_preprocess zeroes
 *     it).  Bits of dq_accum may differ run to run (summation order).
 *   use_atomic = 0: each KV block stores its dQ contribution into its own
 *     workspace slot; a second kernel sums the slots in ascending block order
 *     into dq_accum (fully overwritten).  Bitwise deterministic.
 *   groups == 1: dk, dv [B,S,Hkv,D] bf16 are written here.
 *   groups  > 1: fp32 dK/dV partials (each over groups/P query heads, see
 *     attn_bwd_workspace_bytes) go to the workspace and attn_bwd_postprocess
 *     reduces them; dk and dv are not touched (may be NULL).
 *   workspace/workspace_bytes: at least attn_bwd_workspace_bytes(shape,
 *     causal, use_atomic) bytes; may be NULL when that is 0.
 */
int attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
             const float* lse, const float* delta, float* dq_accum, uint16_t* dk, uint16_t* dv,
             void* workspace, size_t workspace_bytes, attn_shape shape, float softmax_scale,
             int causal, int use_atomic, void* stream);

/*
 * The fixed-order dQ sum that attn_bwd ends with when use_atomic = 0 (the
 * "sum" half of the split+sum template of TileLang #940), on its own:
 * dq_accum[b,h,s,:] = sum over key blocks j = 0 .. J(s), ascending, of the
 * fp32 partials attn_bwd(use_atomic = 0) left in `workspace`, where J(s) is
 * the last key block (causal: the block holding key s).  dq_accum is fully
 * overwritten with the same bits attn_bwd wrote.  For callers that keep the
 * partials and need dQ again, and for timing the two halves of the split
 * path separately.
 *   workspace/workspace_bytes: the buffer of that attn_bwd call, at least
 *     attn_bwd_workspace_bytes(shape, causal, 0) bytes; causal as in it.
 */
int attn_bwd_dq_sum(const void* workspace, size_t workspace_bytes, float* dq_accum, attn_shape shape, int causal,
                    void* stream);

/*
 * attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc).  It runs attn_bwd with use_atomic = 0 (dQ through
 * per-KV-block partials summed in ascending block order: bitwise
 * deterministic) on a scratch array that the library holds in its own code
 * object: 64 MiB of device memory on every GPU the library runs on, kept
 * until the process ends.  The call allocates and frees nothing.
 *   Arguments and outputs as attn_bwd (dq_accum is fully overwritten), with
 *   one difference: dk and dv are always required and always written as
 *   bf16 [B,S,Hkv,D]; for groups > 1 the ascending-r reduction that
 *   attn_bwd_postprocess applies to attn_bwd's partials happens here.  Run
 *   attn_bwd_postprocess(dq_accum, NULL, 0, dq, NULL, NULL, shape with
 *   groups = 1, stream) afterwards for the bf16 dQ.
 *   Scratch needed: (groups > 1 ? 2P/groups : 0) * B*S*Hq*D * 4 bytes plus
 *   ceil(S / bn) * B*S*Hq*D * 4 bytes (P and bn as in
 *   attn_bwd_workspace_bytes);
 *   beyond 64 MiB the call returns
 *   ATTN_ERR_SCRATCH and launches nothing.
 *   The scratch of a GPU is shared by every call on it and holds what the
 *   last call left: calls that may overlap on one GPU (on different streams
 *   or from different threads without ordering) race and give wrong results.
 *   The stream must belong to the current device; the first call on a
 *   device looks up that device's scratch address (hipGetSymbolAddress).
 */
int attn_bwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                     const float* lse, const float* delta, float* dq_accum, uint16_t* dk, uint16_t* dv,
                     attn_shape shape, float softmax_scale, int causal, void* stream);

/*
 * Backward postprocess (flashattn_bwd_postprocess of the TileLang #940
 * examples): dq = bf16(dq_accum) with round-to-nearest-even; for groups > 1
 * also dk/dv[b,s,kv,:] = bf16(sum over p < P, ascending, of the workspace
 * partials [b,s,kv,p]; P as in attn_bwd_workspace_bytes).
 *   dq_accum fp32 [B,Hq,S,D] (input); dq [B,S,Hq,D] bf16 (output);
 *   dk, dv [B,S,Hkv,D] bf16 (outputs, required only when groups > 1);
 *   workspace: the buffer attn_bwd used (required only when groups > 1).
 */
int attn_bwd_postprocess(const float* dq_accum, const void* workspace, size_t workspace_bytes,
                         uint16_t* dq, uint16_t* dk, uint16_t* dv, attn_shape shape, void* stream);

/*
 * Merge of partial results over disjoint key chunks: for every query row,
 *   LSE = ln sum_k exp(LSE_k),   O = sum_k exp(LSE_k - LSE) O_k   (fp32).
 * This is the step context-parallel (ring) attention needs once a query
 * chunk has met every key chunk it can see; the Megatron-LM pull request
 * "TileLang implementation of the fused DSA operations" (NVIDIA Megatron-LM
 * #5049, description, "Packed THD and CP behavior") routes such cases
 * through its common path.  With chunks of equal length every (query chunk,
 * key chunk) pair is an ordinary attn_fwd call (causal for the diagonal
 * pair), and attn_bwd of each pair with the merged LSE and the Delta of the
 * merged O yields that pair's gradient terms.
 *   o_parts  [n_parts][B,S,Hq,D] bf16, contiguous (each part an attn_fwd O)
 *   lse_parts [n_parts][B,Hq,S] fp32 natural log (each part an attn_fwd LSE)
 *   o [B,S,Hq,D] bf16, lse [B,Hq,S] fp32 (outputs; every element written)
 *   n_parts >= 1 (else ATTN_ERR_BAD_SHAPE); shape.groups is not used but
 *   must be valid.
 * Rows whose LSE_k is -inf (no visible key in that part) get weight 0 (their
 * O_k must still be finite, as attn_fwd's zeros are); a row that is -inf in
 * every part gets O = 0 and LSE = -inf.
 */
int attn_merge(const uint16_t* o_parts, const float* lse_parts, int n_parts, uint16_t* o, float* lse,
               attn_shape shape, void* stream);

/*
 * Packed variable-length sequences ("THD" layout).  The rows of all
 * sequences are stored back to back and located by int32 cumulative offsets,
 * the way the cuDNN frontend pull request "CSA: add fused Compressor
 * forward+backward CuTe-DSL kernels (ported from Megatron-LM)" (NVIDIA
 * cudnn-frontend #427, description) passes packs, rows past the last offset
 * being static token-capacity padding.  Sequence b holds query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
 * cu_seqlens_k[b+1]-1 (pass the same array twice when queries and keys are
 * the same tokens).  Attention never crosses sequences: each is ordinary
 * attention of its lq queries over its lk keys, and under causal masking
 * query i (0-based in its sequence) sees key j iff j <= i + lk - lq, i.e.
 * the last query is aligned with the last key (for lq == lk, j <= i).
 *   q, o, dout, dq [Tq,Hq,D] bf16; k, v, dk, dv [Tk,Hkv,D] bf16;
 *   lse, delta [Hq,Tq] fp32; dq_accum [Hq,Tq,D] fp32 (head-major).
 *   cu_seqlens_q/_k: DEVICE memory, n_seqs + 1 int32 each, read by the
 *     kernels (so the host cannot check them).  Each must be non-decreasing
 *     with every length <= its max_seqlen; the kernels clamp every offset to
 *     its tensor and cut a sequence to its first max_seqlen rows, so no access
 *     leaves the tensors whatever they hold, but rows past such a cut count as
 *     padding and overlapping sequences give unspecified results.
 * Query rows that see no key (i < lq - lk under causal masking, lk == 0, or
 * padding) get O = 0, LSE = -inf and dQ = 0; key rows no query sees get
 * dK = dV = 0.  The dout of padding rows is never read by attn_bwd_varlen.
 *
 * Order of calls: attn_fwd_varlen; attn_bwd_preprocess with the dense shape
 * { batch = 1, seqlen = Tq, heads_q, groups, head_dim } (the packed query
 * tensors are exactly that batch-1 problem's); attn_bwd_varlen;
 * attn_bwd_varlen_postprocess.
 */
typedef struct attn_varlen_shape {
  int32_t n_seqs;       /* >= 0 sequences; each cu_seqlens array has n_seqs + 1 entries */
  int32_t total_q;      /* Tq >= 0 query rows of the packed tensors (capacity) */
  int32_t total_k;      /* Tk >= 0 key rows */
  int32_t max_seqlen_q; /* >= 0, bound of every query length (sizes the grid) */
  int32_t max_seqlen_k; /* >= 0, bound of every key length */
  int32_t heads_q;      /* Hq >= 1 */
  int32_t groups;       /* g >= 1, Hq % g == 0 */
  int32_t head_dim;     /* 64 or 128 */
} attn_varlen_shape;

/*
 * Forward over packed sequences: O and LSE of every sequence, attn_fwd's
 * arithmetic per sequence.  Every element of o and lse is written.  With
 * total_q == 0 (after the shape, flag and scale checks) nothing is enqueued
 * and every pointer may be NULL; k and v may be NULL when total_k == 0.
 */
int attn_fwd_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, attn_varlen_shape shape,
                    float softmax_scale, int causal, void* stream);

/*
 * Workspace bytes of attn_bwd_varlen and attn_bwd_varlen_postprocess (0 when
 * none is needed):
 *   groups > 1: fp32 dK and dV partials, [Tk,Hq,D] each;
 *   use_atomic == 0: fp32 dQ partials, [ceil(max_seqlen_k / bn),Hq,Tq,D],
 *     bn as in attn_bwd_workspace_bytes.
 * Returns 0 for an invalid shape.
 */
size_t attn_bwd_varlen_workspace_bytes(attn_varlen_shape shape, int causal, int use_atomic);

/*
 * Backward over packed sequences, with attn_bwd's contract per sequence:
 * dq_accum must be zero on entry when use_atomic = 1 (the preprocess zeroes
 * it) and is fully overwritten when use_atomic = 0 (sums in ascending
 * key-block order, bitwise deterministic); groups == 1 writes dk and dv,
 * groups > 1 writes the workspace partials for attn_bwd_varlen_postprocess.
 * With total_q == total_k == 0 nothing is enqueued and every pointer may be
 * NULL; the query-side pointers may be NULL when total_q == 0, the key-side
 * ones when total_k == 0.
 */
int attn_bwd_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                    const float* lse, const float* delta, float* dq_accum, uint16_t* dk, uint16_t* dv,
                    void* workspace, size_t workspace_bytes, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, attn_varlen_shape shape, float softmax_scale, int causal,
                    int use_atomic, void* stream);

/*
 * Backward postprocess over packed sequences: dq [Tq,Hq,D] = bf16(dq_accum)
 * (RNE); for groups > 1 also dk/dv [Tk,Hkv,D] from the workspace partials of
 * attn_bwd_varlen, summed over each group's query heads in ascending order.
 * Same arguments as attn_bwd_postprocess with the packed shape.
 */
int attn_bwd_varlen_postprocess(const float* dq_accum, const void* workspace, size_t workspace_bytes,
                                uint16_t* dq, uint16_t* dk, uint16_t* dv, attn_varlen_shape shape,
                                void* stream);

/*
 * Simple gated linear attention: chunked backward.  The flash-linear-
 * attention pull request "[Perf] TileLang backends for linear-attention chunk
 * backward (simple_gla / gla / delta_rule / gdn)" (fla-org/flash-linear-
 * attention #1046, summary) speeds up the chunk backward of simple_gla among
 * others; the operation is the standard one, per batch b and head h with the
 * per-token log decay g (natural log; g <= 0 keeps the state bounded) and
 * its running sum G:
 *   o_t = scale * sum_{s<=t} exp(G_t - G_s) (q_t . k_s) v_s
 * and this call returns the gradients of L = sum_t do_t . o_t:
 *   dq_t = scale * sum_{s<=t} exp(G_t - G_s) (do_t . v_s) k_s
 *   dk_s = scale * sum_{t>=s} exp(G_t - G_s) (do_t . v_s) q_t
 *   dv_s = scale * sum_{t>=s} exp(G_t - G_s) (q_t . k_s) do_t
 *   dg_r = sum_{t>=r} (q_t . dq_t - k_t . dk_t)
 * computed in chunks of 64 tokens: one pass over the chunks in each
 * direction carries the chunk state (forward) and its gradient (backward)
 * on chip, fp32 with a bf16 operand copy; the workspace holds only the
 * per-token q.dq and k.dk (fp32) that the gate's reverse running sum reads.
 *   q, k, v, dout, dq, dk, dv [batch, seqlen, heads, 128] bf16 (head_dim 128,
 *     K = V); g, dg [batch, seqlen, heads] fp32 (4-byte aligned).
 *   workspace: at least gla_chunk_bwd_workspace_bytes(shape) bytes.
 * Every element of dq, dk, dv and dg is written.
 */
typedef struct gla_shape {
  int32_t batch;    /* >= 1 */
  int32_t seqlen;   /* T >= 1 (any length; the last chunk may be partial) */
  int32_t heads;    /* >= 1, batch * heads <= 65535 */
  int32_t head_dim; /* 128 */
} gla_shape;

size_t gla_chunk_bwd_workspace_bytes(gla_shape shape);

int gla_chunk_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g, const uint16_t* dout,
                  uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dg, void* workspace, size_t workspace_bytes,
                  gla_shape shape, float scale, void* stream);

/*
 * Sparse MLA attention over top-k gathered latent keys.  The Megatron-LM
 * pull request "TileLang implementation of the fused DSA operations" (NVIDIA
 * Megatron-LM #5049, file table and review summary) adds a sparse MLA
 * forward and backward (with preprocess and postprocess) for 576-wide latent
 * rows whose first 512 channels are the values, index lists with -1 as the
 * unused-slot sentinel, bf16 compute and fp32 accumulation.  Per token t and
 * head h, over the valid entries i of indices[t] (0 <= j < kv_tokens; any
 * other value is an unused slot; a key listed twice counts twice):
 *   s_i = scale * q[t,h] . kv[j_i],   P = softmax(s),
 *   o[t,h] = sum_i P_i kv[j_i, 0:512],   lse[t,h] = ln sum_i exp(s_i)
 * and a token with no valid entry gets o = 0, lse = -inf.
 *   q [tokens, heads, 576] bf16; kv [kv_tokens, 576] bf16 (one latent head
 *   shared by all query heads); indices [tokens, topk] int32 (device);
 *   o [tokens, heads, 512] bf16, lse [tokens, heads] fp32 (outputs; every
 *   element written).  q, kv, o 16-byte aligned; indices and lse 4-byte.
 * Heads are processed in tiles of 32 (a smaller or ragged head count is
 * masked inside the tile).  Errors, all detected on the host before any
 * launch: ATTN_ERR_NULL_PTR, ATTN_ERR_BAD_SHAPE (a size < 1),
 * ATTN_ERR_HEAD_DIM (dims other than 576 / 512), ATTN_ERR_RANGE (topk > 8192,
 * kv_tokens > 524288, tokens * heads * 576 or tokens * topk >= 2^31, a
 * softmax_scale that is not finite and > 0), ATTN_ERR_ALIGN; ATTN_ERR_HIP if
 * the launch fails.  Index values are not checked (they live on the device):
 * anything outside [0, kv_tokens) is an unused slot.
 */
typedef struct smla_shape {
  int32_t tokens;    /* T >= 1 query tokens */
  int32_t kv_tokens; /* Tk, 1 .. 524288 latent rows */
  int32_t heads;     /* H >= 1 query heads */
  int32_t topk;      /* K, 1 .. 8192 index entries per token */
  int32_t dim_qk;    /* 576 */
  int32_t dim_v;     /* 512 */
} smla_shape;

int attn_sparse_mla_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices, uint16_t* o, float* lse,
                        smla_shape shape, float softmax_scale, void* stream);

/*
 * Sparse MLA backward, the same preprocess / backward / postprocess split as
 * the dense path (the gradients of sum o . dout):
 *   preprocess: delta[t,h] = sum_{d<512} o[t,h,d] dout[t,h,d] (fp32
 *     [tokens, heads]); dkv_accum (fp32 [kv_tokens, 576], may be NULL) is
 *     set to zero.
 *   backward: with P and dS = P (dP - delta) recomputed from q, kv, lse,
 *     dP_i = dout[t,h] . kv[j_i, 0:512]:
 *       dq[t,h]      = scale * sum_i dS_i kv[j_i]         (bf16, written)
 *       dkv_accum[j_i] += scale * sum_h dS_i q[t,h], and its first 512
 *                         channels += sum_h P_i dout[t,h]  (fp32 atomic adds
 *                         of each token's 32-head tile; must hold zeros or a
 *                         running sum on entry; the order of the additions,
 *                         and so the last bits, may differ run to run)
 *   postprocess: dkv = bf16(dkv_accum) (RNE), [kv_tokens, 576].
 * lse is the forward's.  Arguments otherwise as attn_sparse_mla_fwd
 * (dout [tokens, heads, 512] bf16; dq 16-byte aligned; delta 4-byte).
 */
int attn_sparse_mla_bwd_preprocess(const uint16_t* o, const uint16_t* dout, float* delta, float* dkv_accum,
                                   smla_shape shape, void* stream);
int attn_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const uint16_t* dout, const int32_t* indices,
                        const float* lse, const float* delta, uint16_t* dq, float* dkv_accum, smla_shape shape,
                        float softmax_scale, void* stream);
int attn_sparse_mla_bwd_postprocess(const float* dkv_accum, uint16_t* dkv, smla_shape shape, void* stream);

/*
 * Sparse MLA backward with a deterministic dKV (bitwise reproducible run to
 * run), the alternative to fp32 atomics that the cuDNN frontend pull request
 * "CSA: add fused Compressor forward+backward CuTe-DSL kernels (ported from
 * Megatron-LM)" (NVIDIA cudnn-frontend #427, numerics and determinism
 * section) names: partials reduced in a fixed order.  Takes the place of
 * attn_sparse_mla_bwd + attn_sparse_mla_bwd_postprocess (run
 * attn_sparse_mla_bwd_preprocess first, dkv_accum may be NULL there):
 *   dq  [tokens, heads, 576] bf16, written, as attn_sparse_mla_bwd;
 *   dkv [kv_tokens, 576] bf16, written whole: row j is the bf16 (RNE) of
 *       the sum, over the valid entries (t, i) with indices[t, i] = j and
 *       over the 32-head tiles of t, of scale * sum_h dS q[t,h] (+ sum_h
 *       P dout[t,h] in channels 0..511), each entry's fp32 row formed
 *       whole and the rows added in one fixed order that depends on the
 *       index lists alone (rows ordered by token, slot and head tile, summed
 *       in four interleaved running sums that are then added in a fixed
 *       order); 0 for a row no valid entry names.
 * workspace: device memory of at least
 * attn_sparse_mla_bwd_split_workspace_bytes(shape) bytes, 16-byte aligned,
 * owned by the caller, no initial contents needed; its size is dominated by
 * one fp32 row of 576 per entry slot and 32-head tile
 * (tokens * topk * ceil(heads / 32) * 2304 bytes).  Errors as
 * attn_sparse_mla_bwd, plus ATTN_ERR_WORKSPACE (NULL or too small).
 * attn_sparse_mla_bwd_split_workspace_bytes returns 0 for an invalid shape.
 */
size_t attn_sparse_mla_bwd_split_workspace_bytes(smla_shape shape);
int attn_sparse_mla_bwd_split(const uint16_t* q, const uint16_t* kv, const uint16_t* dout, const int32_t* indices,
                              const float* lse, const float* delta, uint16_t* dq, uint16_t* dkv, void* workspace,
                              size_t workspace_bytes, smla_shape shape, float softmax_scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MI355_ATTN_H */
