// C ABI of libmi355_attn.so: argument validation on the host, then kernel
// launches on the caller's stream.  Every check runs before anything is
// enqueued; the library never allocates, frees or synchronises.
#include <math.h>

#include "kernels.h"
#include "mi355_attn.h"

using namespace mi355;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(const attn_shape& s) {
  if (s.batch < 1 || s.seqlen < 1 || s.heads_q < 1 || s.groups < 1) return ATTN_ERR_BAD_SHAPE;
  if (s.heads_q % s.groups) return ATTN_ERR_BAD_SHAPE;
  if (s.head_dim != 64 && s.head_dim != 128) return ATTN_ERR_HEAD_DIM;
  const long long nq = (long long)s.batch * s.seqlen * s.heads_q * s.head_dim;
  if (nq >= (1LL << 31)) return ATTN_ERR_RANGE;
  // Kernels address up to 256 rows of one head with 32-bit byte offsets.
  if ((long long)s.heads_q * s.head_dim > (1LL << 22)) return ATTN_ERR_RANGE;
  return ATTN_OK;
}

bool good_scale(float x) { return isfinite(x) && x > 0.f; }

size_t elems_q(const attn_shape& s) { return (size_t)s.batch * s.seqlen * s.heads_q * s.head_dim; }
int n_key_blocks(const attn_shape& s) { return (s.seqlen + kBwdBlockN - 1) / kBwdBlockN; }

// Workspace layout: [dK partials | dV partials] when groups > 1, then the
// split path's dQ partials.  Every region is a multiple of 256 bytes.
size_t ws_gqa_bytes(const attn_shape& s) { return s.groups > 1 ? 2 * elems_q(s) * sizeof(float) : 0; }
size_t ws_split_bytes(const attn_shape& s, int use_atomic) {
  return use_atomic ? 0 : (size_t)n_key_blocks(s) * elems_q(s) * sizeof(float);
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Packed sequences: the same limits as the dense batch-1 problem of T rows.
int check_varlen(const attn_varlen_shape& s) {
  if (s.n_seqs < 0 || s.total < 0 || s.max_seqlen < 0 || s.heads_q < 1 || s.groups < 1) return ATTN_ERR_BAD_SHAPE;
  if (s.heads_q % s.groups) return ATTN_ERR_BAD_SHAPE;
  if (s.head_dim != 64 && s.head_dim != 128) return ATTN_ERR_HEAD_DIM;
  if ((long long)s.total * s.heads_q * s.head_dim >= (1LL << 31)) return ATTN_ERR_RANGE;
  if ((long long)s.heads_q * s.head_dim > (1LL << 22)) return ATTN_ERR_RANGE;
  // Grid: n_seqs * heads * ceil(max_seqlen / 32) workgroups must fit 32 bits.
  if ((long long)s.n_seqs * s.heads_q * ((s.max_seqlen + 31) / 32) >= (1LL << 31)) return ATTN_ERR_RANGE;
  return ATTN_OK;
}

size_t elems_varlen(const attn_varlen_shape& s) { return (size_t)s.total * s.heads_q * s.head_dim; }
size_t ws_varlen_gqa_bytes(const attn_varlen_shape& s) { return s.groups > 1 ? 2 * elems_varlen(s) * 4 : 0; }
size_t ws_varlen_split_bytes(const attn_varlen_shape& s, int use_atomic) {
  const int nblk = (s.max_seqlen + kBwdBlockN - 1) / kBwdBlockN;
  return use_atomic ? 0 : (size_t)nblk * elems_varlen(s) * 4;
}

}  // namespace

extern "C" {

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL_PTR: return "a required pointer is NULL";
    case ATTN_ERR_BAD_SHAPE: return "invalid shape: sizes must be >= 1 and heads_q a multiple of groups";
    case ATTN_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case ATTN_ERR_ALIGN: return "tensor base pointers must be 16-byte aligned";
    case ATTN_ERR_RANGE:
      return "out of range: a tensor has >= 2^31 elements, heads_q * head_dim > 2^22, or softmax_scale is not "
             "finite and > 0";
    case ATTN_ERR_WORKSPACE: return "workspace is NULL or smaller than attn_bwd_workspace_bytes()";
    case ATTN_ERR_HIP: return "HIP runtime reported a launch error";
    case ATTN_ERR_FLAG: return "causal and use_atomic must be 0 or 1";
    default: return "unknown status";
  }
}

int attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
             attn_shape shape, float softmax_scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL_PTR;
  const int st = check_shape(shape);
  if (st) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_FLAG;
  if (!good_scale(softmax_scale)) return ATTN_ERR_RANGE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;
  FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = shape.batch;
  p.S = shape.seqlen;
  p.Hq = shape.heads_q;
  p.G = shape.groups;
  p.Hkv = shape.heads_q / shape.groups;
  p.D = shape.head_dim;
  p.scale = softmax_scale;
  p.causal = causal;
  p.cu = nullptr;
  p.T = 0;
  return hip_status(launch_fwd(p, (hipStream_t)stream));
}

int attn_bwd_preprocess(const uint16_t* o, const uint16_t* dout, float* delta, float* dq_accum,
                        attn_shape shape, void* stream) {
  if (!o || !dout || !delta) return ATTN_ERR_NULL_PTR;
  const int st = check_shape(shape);
  if (st) return st;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(delta) || (dq_accum && !aligned16(dq_accum)))
    return ATTN_ERR_ALIGN;
  return hip_status(launch_preprocess(o, dout, delta, dq_accum, shape.batch, shape.seqlen, shape.heads_q,
                                      shape.head_dim, (hipStream_t)stream));
}

size_t attn_bwd_workspace_bytes(attn_shape shape, int causal, int use_atomic) {
  if (check_shape(shape) != ATTN_OK) return 0;
  if ((causal != 0 && causal != 1) || (use_atomic != 0 && use_atomic != 1)) return 0;
  return ws_gqa_bytes(shape) + ws_split_bytes(shape, use_atomic);
}

int attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout, const float* lse,
             const float* delta, float* dq_accum, uint16_t* dk, uint16_t* dv, void* workspace,
             size_t workspace_bytes, attn_shape shape, float softmax_scale, int causal, int use_atomic,
             void* stream) {
  if (!q || !k || !v || !dout || !lse || !delta || !dq_accum) return ATTN_ERR_NULL_PTR;
  const int st = check_shape(shape);
  if (st) return st;
  if ((causal != 0 && causal != 1) || (use_atomic != 0 && use_atomic != 1)) return ATTN_ERR_FLAG;
  if (shape.groups == 1 && (!dk || !dv)) return ATTN_ERR_NULL_PTR;
  if (!good_scale(softmax_scale)) return ATTN_ERR_RANGE;
  const size_t need = ws_gqa_bytes(shape) + ws_split_bytes(shape, use_atomic);
  if (need && (!workspace || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(lse) ||
      !aligned16(delta) || !aligned16(dq_accum) || (dk && !aligned16(dk)) || (dv && !aligned16(dv)) ||
      (workspace && !aligned16(workspace)))
    return ATTN_ERR_ALIGN;

  BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.dout = dout;
  p.lse = lse;
  p.delta = delta;
  p.dq_accum = dq_accum;
  p.dk = dk;
  p.dv = dv;
  char* ws = (char*)workspace;
  const size_t nq_bytes = elems_q(shape) * sizeof(float);
  p.dk_part = shape.groups > 1 ? (float*)ws : nullptr;
  p.dv_part = shape.groups > 1 ? (float*)(ws + nq_bytes) : nullptr;
  p.dq_part = use_atomic ? nullptr : (float*)(ws + ws_gqa_bytes(shape));
  p.B = shape.batch;
  p.S = shape.seqlen;
  p.Hq = shape.heads_q;
  p.G = shape.groups;
  p.Hkv = shape.heads_q / shape.groups;
  p.D = shape.head_dim;
  p.scale = softmax_scale;
  p.log2_scale = log2f(softmax_scale);
  p.causal = causal;
  p.use_atomic = use_atomic;
  p.cu = nullptr;
  p.T = 0;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_bwd(p, s);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  if (!use_atomic)
    e = launch_dq_sum(p.dq_part, dq_accum, p.B, p.S, p.Hq, p.D, causal, s);
  return hip_status(e);
}

int attn_bwd_postprocess(const float* dq_accum, const void* workspace, size_t workspace_bytes, uint16_t* dq,
                         uint16_t* dk, uint16_t* dv, attn_shape shape, void* stream) {
  if (!dq_accum || !dq) return ATTN_ERR_NULL_PTR;
  const int st = check_shape(shape);
  if (st) return st;
  const bool gqa = shape.groups > 1;
  if (gqa && (!dk || !dv)) return ATTN_ERR_NULL_PTR;
  if (gqa && (!workspace || workspace_bytes < ws_gqa_bytes(shape))) return ATTN_ERR_WORKSPACE;
  if (!aligned16(dq_accum) || !aligned16(dq) || (gqa && (!aligned16(dk) || !aligned16(dv) || !aligned16(workspace))))
    return ATTN_ERR_ALIGN;
  const char* ws = (const char*)workspace;
  const size_t nq_bytes = elems_q(shape) * sizeof(float);
  return hip_status(launch_postprocess(dq_accum, gqa ? (const float*)ws : nullptr,
                                       gqa ? (const float*)(ws + nq_bytes) : nullptr, dq, gqa ? dk : nullptr,
                                       gqa ? dv : nullptr, shape.batch, shape.seqlen, shape.heads_q,
                                       shape.groups, shape.head_dim, (hipStream_t)stream));
}

int attn_merge(const uint16_t* o_parts, const float* lse_parts, int n_parts, uint16_t* o, float* lse,
               attn_shape shape, void* stream) {
  if (!o_parts || !lse_parts || !o || !lse) return ATTN_ERR_NULL_PTR;
  if (n_parts < 1) return ATTN_ERR_BAD_SHAPE;
  const int st = check_shape(shape);
  if (st) return st;
  if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;
  return hip_status(launch_merge(o_parts, lse_parts, n_parts, o, lse, shape.batch, shape.seqlen, shape.heads_q,
                                 shape.head_dim, (hipStream_t)stream));
}

int attn_fwd_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                    const int32_t* cu_seqlens, attn_varlen_shape shape, float softmax_scale, int causal,
                    void* stream) {
  const int st = check_varlen(shape);
  if (st) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_FLAG;
  if (!good_scale(softmax_scale)) return ATTN_ERR_RANGE;
  if (shape.total == 0) return ATTN_OK;  // no rows: nothing to do, pointers unused
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return ATTN_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (shape.n_seqs > 0 && shape.max_seqlen > 0) {
    FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.cu = cu_seqlens;
    p.T = shape.total;
    p.B = shape.n_seqs;
    p.S = shape.max_seqlen;
    p.Hq = shape.heads_q;
    p.G = shape.groups;
    p.Hkv = shape.heads_q / shape.groups;
    p.D = shape.head_dim;
    p.scale = softmax_scale;
    p.causal = causal;
    const hipError_t e = launch_fwd(p, s);
    if (e != hipSuccess) return ATTN_ERR_HIP;
  }
  return hip_status(launch_pad_fill(o, nullptr, 0, shape.heads_q, lse, shape.heads_q, -INFINITY, cu_seqlens,
                                    shape.n_seqs, shape.total, shape.max_seqlen, shape.head_dim, s));
}

size_t attn_bwd_varlen_workspace_bytes(attn_varlen_shape shape, int causal, int use_atomic) {
  if (check_varlen(shape) != ATTN_OK) return 0;
  if ((causal != 0 && causal != 1) || (use_atomic != 0 && use_atomic != 1)) return 0;
  return ws_varlen_gqa_bytes(shape) + ws_varlen_split_bytes(shape, use_atomic);
}

int attn_bwd_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                    const float* lse, const float* delta, float* dq_accum, uint16_t* dk, uint16_t* dv,
                    void* workspace, size_t workspace_bytes, const int32_t* cu_seqlens,
                    attn_varlen_shape shape, float softmax_scale, int causal, int use_atomic, void* stream) {
  const int st = check_varlen(shape);
  if (st) return st;
  if ((causal != 0 && causal != 1) || (use_atomic != 0 && use_atomic != 1)) return ATTN_ERR_FLAG;
  if (!good_scale(softmax_scale)) return ATTN_ERR_RANGE;
  if (shape.total == 0) return ATTN_OK;  // no rows: nothing to do, pointers unused
  if (!q || !k || !v || !dout || !lse || !delta || !dq_accum || !cu_seqlens) return ATTN_ERR_NULL_PTR;
  if (shape.groups == 1 && (!dk || !dv)) return ATTN_ERR_NULL_PTR;
  const size_t need = ws_varlen_gqa_bytes(shape) + ws_varlen_split_bytes(shape, use_atomic);
  if (need && (!workspace || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(lse) ||
      !aligned16(delta) || !aligned16(dq_accum) || (dk && !aligned16(dk)) || (dv && !aligned16(dv)) ||
      (workspace && !aligned16(workspace)))
    return ATTN_ERR_ALIGN;

  BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.dout = dout;
  p.lse = lse;
  p.delta = delta;
  p.dq_accum = dq_accum;
  p.dk = dk;
  p.dv = dv;
  char* ws = (char*)workspace;
  const size_t nq_bytes = elems_varlen(shape) * sizeof(float);
  const bool gqa = shape.groups > 1;
  p.dk_part = gqa ? (float*)ws : nullptr;
  p.dv_part = gqa ? (float*)(ws + nq_bytes) : nullptr;
  p.dq_part = use_atomic ? nullptr : (float*)(ws + ws_varlen_gqa_bytes(shape));
  p.cu = cu_seqlens;
  p.T = shape.total;
  p.B = shape.n_seqs;
  p.S = shape.max_seqlen;
  p.Hq = shape.heads_q;
  p.G = shape.groups;
  p.Hkv = shape.heads_q / shape.groups;
  p.D = shape.head_dim;
  p.scale = softmax_scale;
  p.log2_scale = log2f(softmax_scale);
  p.causal = causal;
  p.use_atomic = use_atomic;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  const bool any = shape.n_seqs > 0 && shape.max_seqlen > 0;
  if (any) e = launch_bwd(p, s);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  // Padding rows: zero dK/dV (the fp32 partials when groups > 1).
  e = gqa ? launch_pad_fill(p.dk_part, p.dv_part, 1, shape.heads_q, nullptr, shape.heads_q, 0.f, cu_seqlens,
                            shape.n_seqs, shape.total, shape.max_seqlen, shape.head_dim, s)
          : launch_pad_fill(dk, dv, 0, p.Hkv, nullptr, shape.heads_q, 0.f, cu_seqlens, shape.n_seqs, shape.total,
                            shape.max_seqlen, shape.head_dim, s);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  if (!use_atomic)
    e = launch_dq_sum_varlen(p.dq_part, dq_accum, cu_seqlens, shape.n_seqs, shape.total, shape.max_seqlen,
                             shape.heads_q, shape.head_dim, causal, s);
  return hip_status(e);
}

}  // extern "C"
