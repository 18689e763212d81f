// C ABI of libmi355_attn.so: argument validation on the host, then kernel
// launches on the caller's stream.  Every check runs before anything is
// enqueued; the library never allocates, frees or synchronises.
#include <math.h>

#include <mutex>

#include "kernels.h"
#include "mi355_attn.h"
#include "smla_split.h"

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
int n_key_blocks(const attn_shape& s) {
  const int bn = bwd_block_n(s.head_dim);
  return (s.seqlen + bn - 1) / bn;
}

// Grouped queries: fp32 dK/dV partials per (key row, KV head).
int gqa_parts(const attn_shape& s) {
  return bwd_gqa_parts(s.batch, s.heads_q / s.groups, s.groups, s.seqlen, s.head_dim);
}
// Workspace layout: [dK partials | dV partials] when groups > 1, then the
// split path's dQ partials.  Every region is a multiple of 256 bytes.
size_t ws_gqa_half_bytes(const attn_shape& s) {
  return s.groups > 1 ? elems_q(s) / s.groups * gqa_parts(s) * sizeof(float) : 0;
}
size_t ws_gqa_bytes(const attn_shape& s) { return 2 * ws_gqa_half_bytes(s); }
size_t ws_split_bytes(const attn_shape& s, int use_atomic) {
  return use_atomic ? 0 : (size_t)n_key_blocks(s) * elems_q(s) * sizeof(float);
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Packed sequences: the same limits as the dense batch-1 problems of Tq
// query rows and Tk key rows.
int check_varlen(const attn_varlen_shape& s) {
  if (s.n_seqs < 0 || s.total_q < 0 || s.total_k < 0 || s.max_seqlen_q < 0 || s.max_seqlen_k < 0 ||
      s.heads_q < 1 || s.groups < 1)
    return ATTN_ERR_BAD_SHAPE;
  if (s.heads_q % s.groups) return ATTN_ERR_BAD_SHAPE;
  if (s.head_dim != 64 && s.head_dim != 128) return ATTN_ERR_HEAD_DIM;
  const long long hd = (long long)s.heads_q * s.head_dim;
  if ((long long)s.total_q * hd >= (1LL << 31) || (long long)s.total_k * hd >= (1LL << 31)) return ATTN_ERR_RANGE;
  if (hd > (1LL << 22)) return ATTN_ERR_RANGE;
  // Grids: n_seqs * heads * ceil(max_seqlen / 32) workgroups must fit 32 bits.
  const long long blk = (long long)((s.max_seqlen_q > s.max_seqlen_k ? s.max_seqlen_q : s.max_seqlen_k) + 31) / 32;
  if ((long long)s.n_seqs * s.heads_q * blk >= (1LL << 31)) return ATTN_ERR_RANGE;
  return ATTN_OK;
}

// Varlen workspace: [dK partials | dV partials] ([Tk][Hq][D] fp32 each) when
// groups > 1, then the split path's dQ partials ([n_kv_blocks][Hq][Tq][D]).
size_t ws_varlen_gqa_bytes(const attn_varlen_shape& s) {
  return s.groups > 1 ? 2 * (size_t)s.total_k * s.heads_q * s.head_dim * 4 : 0;
}
size_t ws_varlen_split_bytes(const attn_varlen_shape& s, int use_atomic) {
  const int bn = bwd_block_n(s.head_dim), nblk = (s.max_seqlen_k + bn - 1) / bn;
  return use_atomic ? 0 : (size_t)nblk * s.total_q * s.heads_q * s.head_dim * 4;
}

// Sequences with rows on both sides exist: the main kernels have work.
bool varlen_any(const attn_varlen_shape& s) { return s.n_seqs > 0 && s.max_seqlen_q > 0 && s.max_seqlen_k > 0; }

int check_gla(const gla_shape& s) {
  if (s.batch < 1 || s.seqlen < 1 || s.heads < 1) return ATTN_ERR_BAD_SHAPE;
  if (s.head_dim != 128) return ATTN_ERR_HEAD_DIM;
  if ((long long)s.batch * s.seqlen * s.heads * s.head_dim >= (1LL << 31)) return ATTN_ERR_RANGE;
  if ((long long)s.batch * s.heads > 65535) return ATTN_ERR_RANGE;  // grid y of the chunk stage
  return ATTN_OK;
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int check_smla(const smla_shape& s) {
  if (s.tokens < 1 || s.kv_tokens < 1 || s.heads < 1 || s.topk < 1) return ATTN_ERR_BAD_SHAPE;
  if (s.dim_qk != 576 || s.dim_v != 512) return ATTN_ERR_HEAD_DIM;
  if ((long long)s.tokens * s.heads * 576 >= (1LL << 31) || s.kv_tokens > kSmlaMaxKvTokens ||
      (long long)s.tokens * s.topk >= (1LL << 31) || s.topk > 8192)
    return ATTN_ERR_RANGE;
  return ATTN_OK;
}

// Scratch of attn_bwd_noalloc: a fixed device array in the library's code
// object, one copy per GPU for the life of the process.  On the host its
// name stands for a host-side shadow, so kernels get the device address
// hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kScratchBytes = 64u << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return ATTN_ERR_HIP;
    scratch_ptr[dev] = ptr;
  }
  *out = (char*)scratch_ptr[dev];
  return ATTN_OK;
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
    case ATTN_ERR_SCRATCH: return "problem needs more than the library's fixed 64 MiB scratch array";
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
  p.cu_k = nullptr;
  p.T = p.Tk = 0;
  p.Sk = shape.seqlen;
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
  p.dk_part = shape.groups > 1 ? (float*)ws : nullptr;
  p.dv_part = shape.groups > 1 ? (float*)(ws + ws_gqa_half_bytes(shape)) : nullptr;
  p.hpw = shape.groups / gqa_parts(shape);
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
  p.cu_k = nullptr;
  p.T = p.Tk = 0;
  p.Sk = shape.seqlen;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_bwd(p, s);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  if (!use_atomic)
    e = launch_dq_sum(p.dq_part, dq_accum, p.B, p.S, p.Hq, p.D, causal, s);
  return hip_status(e);
}

int attn_bwd_dq_sum(const void* workspace, size_t workspace_bytes, float* dq_accum, attn_shape shape, int causal,
                    void* stream) {
  if (!workspace || !dq_accum) return ATTN_ERR_NULL_PTR;
  const int st = check_shape(shape);
  if (st) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_FLAG;
  if (workspace_bytes < ws_gqa_bytes(shape) + ws_split_bytes(shape, 0)) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(dq_accum)) return ATTN_ERR_ALIGN;
  const float* part = (const float*)((const char*)workspace + ws_gqa_bytes(shape));
  return hip_status(launch_dq_sum(part, dq_accum, shape.batch, shape.seqlen, shape.heads_q, shape.head_dim, causal,
                                  (hipStream_t)stream));
}

int attn_bwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                     const float* lse, const float* delta, float* dq_accum, uint16_t* dk, uint16_t* dv,
                     attn_shape shape, float softmax_scale, int causal, void* stream) {
  if (!q || !k || !v || !dout || !lse || !delta || !dq_accum || !dk || !dv) return ATTN_ERR_NULL_PTR;
  const int st = check_shape(shape);
  if (st) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_FLAG;
  if (!good_scale(softmax_scale)) return ATTN_ERR_RANGE;
  const size_t need = ws_gqa_bytes(shape) + ws_split_bytes(shape, 0);
  if (need > kScratchBytes) return ATTN_ERR_SCRATCH;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(lse) ||
      !aligned16(delta) || !aligned16(dq_accum) || !aligned16(dk) || !aligned16(dv))
    return ATTN_ERR_ALIGN;
  char* ws = nullptr;
  const int sst = scratch_of_current_device(&ws);
  if (sst) return sst;
  // attn_bwd's split path on the scratch array.  Every scratch element a
  // kernel reads was written earlier in this call, so nothing is cleared.
  const int bst = attn_bwd(q, k, v, dout, lse, delta, dq_accum, dk, dv, ws, kScratchBytes, shape, softmax_scale,
                           causal, 0, stream);
  if (bst || shape.groups == 1) return bst;
  return hip_status(launch_gqa_reduce((const float*)ws, (const float*)(ws + ws_gqa_half_bytes(shape)), dk, dv,
                                      shape.seqlen, shape.heads_q, shape.heads_q / shape.groups, gqa_parts(shape),
                                      shape.head_dim, (long long)shape.batch * shape.seqlen, (hipStream_t)stream));
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
  return hip_status(launch_postprocess(dq_accum, gqa ? (const float*)ws : nullptr,
                                       gqa ? (const float*)(ws + ws_gqa_half_bytes(shape)) : nullptr, dq,
                                       gqa ? dk : nullptr, gqa ? dv : nullptr, shape.batch, shape.seqlen,
                                       shape.heads_q, shape.heads_q / shape.groups, gqa ? gqa_parts(shape) : 1,
                                       shape.head_dim, (long long)shape.batch * shape.seqlen, (hipStream_t)stream));
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
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, attn_varlen_shape shape,
                    float softmax_scale, int causal, void* stream) {
  const int st = check_varlen(shape);
  if (st) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_FLAG;
  if (!good_scale(softmax_scale)) return ATTN_ERR_RANGE;
  if (shape.total_q == 0) return ATTN_OK;  // no query rows: nothing to do, pointers unused
  if (!q || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL_PTR;
  if (shape.total_k > 0 && (!k || !v)) return ATTN_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (shape.total_k > 0 && varlen_any(shape)) {
    FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.cu = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.T = shape.total_q;
    p.Tk = shape.total_k;
    p.B = shape.n_seqs;
    p.S = shape.max_seqlen_q;
    p.Sk = shape.max_seqlen_k;
    p.Hq = shape.heads_q;
    p.G = shape.groups;
    p.Hkv = shape.heads_q / shape.groups;
    p.D = shape.head_dim;
    p.scale = softmax_scale;
    p.causal = causal;
    const hipError_t e = launch_fwd(p, s);
    if (e != hipSuccess) return ATTN_ERR_HIP;
    // Rows inside a sequence are all written by the kernel (O = 0 and
    // LSE = -inf where no key is visible); the rest is padding.
    return hip_status(launch_pad_fill(o, nullptr, 0, shape.heads_q, lse, shape.heads_q, -INFINITY, cu_seqlens_q,
                                      shape.n_seqs, shape.total_q, shape.max_seqlen_q, shape.head_dim, s));
  }
  // No key anywhere: every query row is empty.
  return hip_status(launch_pad_fill(o, nullptr, 0, shape.heads_q, lse, shape.heads_q, -INFINITY, cu_seqlens_q, 0,
                                    shape.total_q, 0, shape.head_dim, s));
}

size_t attn_bwd_varlen_workspace_bytes(attn_varlen_shape shape, int causal, int use_atomic) {
  if (check_varlen(shape) != ATTN_OK) return 0;
  if ((causal != 0 && causal != 1) || (use_atomic != 0 && use_atomic != 1)) return 0;
  return ws_varlen_gqa_bytes(shape) + ws_varlen_split_bytes(shape, use_atomic);
}

int attn_bwd_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                    const float* lse, const float* delta, float* dq_accum, uint16_t* dk, uint16_t* dv,
                    void* workspace, size_t workspace_bytes, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, attn_varlen_shape shape, float softmax_scale, int causal,
                    int use_atomic, void* stream) {
  const int st = check_varlen(shape);
  if (st) return st;
  if ((causal != 0 && causal != 1) || (use_atomic != 0 && use_atomic != 1)) return ATTN_ERR_FLAG;
  if (!good_scale(softmax_scale)) return ATTN_ERR_RANGE;
  if (shape.total_q == 0 && shape.total_k == 0) return ATTN_OK;  // no rows: nothing to do, pointers unused
  if (!cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL_PTR;
  if (shape.total_q > 0 && (!q || !dout || !lse || !delta || !dq_accum)) return ATTN_ERR_NULL_PTR;
  if (shape.total_k > 0 && (!k || !v)) return ATTN_ERR_NULL_PTR;
  if (shape.total_k > 0 && shape.groups == 1 && (!dk || !dv)) return ATTN_ERR_NULL_PTR;
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
  const bool gqa = shape.groups > 1;
  const size_t nkv_bytes = (size_t)shape.total_k * shape.heads_q * shape.head_dim * sizeof(float);
  p.dk_part = gqa ? (float*)ws : nullptr;
  p.dv_part = gqa ? (float*)(ws + nkv_bytes) : nullptr;
  p.dq_part = use_atomic ? nullptr : (float*)(ws + ws_varlen_gqa_bytes(shape));
  p.hpw = 1;  // one query head per workgroup: each leaves its own partial
  p.cu = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.T = shape.total_q;
  p.Tk = shape.total_k;
  p.B = shape.n_seqs;
  p.S = shape.max_seqlen_q;
  p.Sk = shape.max_seqlen_k;
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
  const bool run = shape.total_q > 0 && shape.total_k > 0 && varlen_any(shape);
  if (run) e = launch_bwd(p, s);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  // Key rows outside every sequence (all of them when the kernel had no
  // work): zero dK/dV (the fp32 partials when groups > 1).
  if (shape.total_k > 0) {
    const int ns = run ? shape.n_seqs : 0;
    e = gqa ? launch_pad_fill(p.dk_part, p.dv_part, 1, shape.heads_q, nullptr, shape.heads_q, 0.f, cu_seqlens_k,
                              ns, shape.total_k, shape.max_seqlen_k, shape.head_dim, s)
            : launch_pad_fill(dk, dv, 0, p.Hkv, nullptr, shape.heads_q, 0.f, cu_seqlens_k, ns, shape.total_k,
                              shape.max_seqlen_k, shape.head_dim, s);
    if (e != hipSuccess) return ATTN_ERR_HIP;
  }
  if (!use_atomic && shape.total_q > 0)
    e = launch_dq_sum_varlen(p.dq_part, dq_accum, cu_seqlens_q, cu_seqlens_k, shape.n_seqs, shape.total_q,
                             shape.total_k, shape.max_seqlen_q, shape.max_seqlen_k, shape.heads_q, shape.head_dim,
                             causal, s);
  return hip_status(e);
}

int attn_bwd_varlen_postprocess(const float* dq_accum, const void* workspace, size_t workspace_bytes,
                                uint16_t* dq, uint16_t* dk, uint16_t* dv, attn_varlen_shape shape,
                                void* stream) {
  const int st = check_varlen(shape);
  if (st) return st;
  const bool gqa = shape.groups > 1 && shape.total_k > 0;
  if (shape.total_q == 0 && !gqa) return ATTN_OK;  // nothing to convert, pointers unused
  if (shape.total_q > 0 && (!dq_accum || !dq)) return ATTN_ERR_NULL_PTR;
  if (gqa && (!dk || !dv)) return ATTN_ERR_NULL_PTR;
  if (gqa && (!workspace || workspace_bytes < ws_varlen_gqa_bytes(shape))) return ATTN_ERR_WORKSPACE;
  if (!aligned16(dq_accum) || !aligned16(dq) || (gqa && (!aligned16(dk) || !aligned16(dv) || !aligned16(workspace))))
    return ATTN_ERR_ALIGN;
  const char* ws = (const char*)workspace;
  const size_t nkv_bytes = (size_t)shape.total_k * shape.heads_q * shape.head_dim * sizeof(float);
  return hip_status(launch_postprocess(dq_accum, gqa ? (const float*)ws : nullptr,
                                       gqa ? (const float*)(ws + nkv_bytes) : nullptr, dq, gqa ? dk : nullptr,
                                       gqa ? dv : nullptr, 1, shape.total_q, shape.heads_q,
                                       shape.heads_q / shape.groups, gqa ? shape.groups : 1, shape.head_dim,
                                       shape.total_k, (hipStream_t)stream));
}

size_t gla_chunk_bwd_workspace_bytes(gla_shape shape) {
  if (check_gla(shape) != ATTN_OK) return 0;
  return gla_bwd_workspace_bytes(shape.batch, shape.seqlen, shape.heads);
}

int gla_chunk_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g, const uint16_t* dout,
                  uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dg, void* workspace, size_t workspace_bytes,
                  gla_shape shape, float scale, void* stream) {
  if (!q || !k || !v || !g || !dout || !dq || !dk || !dv || !dg) return ATTN_ERR_NULL_PTR;
  const int st = check_gla(shape);
  if (st) return st;
  if (!good_scale(scale)) return ATTN_ERR_RANGE;
  if (!workspace || workspace_bytes < gla_bwd_workspace_bytes(shape.batch, shape.seqlen, shape.heads))
    return ATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || !aligned16(workspace) || !aligned4(g) || !aligned4(dg))
    return ATTN_ERR_ALIGN;
  return hip_status(launch_gla_bwd(q, k, v, dout, g, dq, dk, dv, dg, workspace, shape.batch, shape.seqlen,
                                   shape.heads, scale, (hipStream_t)stream));
}

int attn_sparse_mla_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices, uint16_t* o, float* lse,
                        smla_shape shape, float softmax_scale, void* stream) {
  if (!q || !kv || !indices || !o || !lse) return ATTN_ERR_NULL_PTR;
  const int st = check_smla(shape);
  if (st) return st;
  if (!good_scale(softmax_scale)) return ATTN_ERR_RANGE;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(o) || !aligned4(lse) || !aligned4(indices)) return ATTN_ERR_ALIGN;
  return hip_status(launch_smla_fwd(q, kv, indices, o, lse, shape.tokens, shape.kv_tokens, shape.heads, shape.topk,
                                    softmax_scale, (hipStream_t)stream));
}

int attn_sparse_mla_bwd_preprocess(const uint16_t* o, const uint16_t* dout, float* delta, float* dkv_accum,
                                   smla_shape shape, void* stream) {
  if (!o || !dout || !delta) return ATTN_ERR_NULL_PTR;
  const int st = check_smla(shape);
  if (st) return st;
  if (!aligned16(o) || !aligned16(dout) || !aligned4(delta) || (dkv_accum && !aligned16(dkv_accum)))
    return ATTN_ERR_ALIGN;
  return hip_status(launch_smla_bwd_pre(o, dout, delta, dkv_accum, shape.tokens, shape.kv_tokens, shape.heads,
                                        (hipStream_t)stream));
}

int attn_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const uint16_t* dout, const int32_t* indices,
                        const float* lse, const float* delta, uint16_t* dq, float* dkv_accum, smla_shape shape,
                        float softmax_scale, void* stream) {
  if (!q || !kv || !dout || !indices || !lse || !delta || !dq || !dkv_accum) return ATTN_ERR_NULL_PTR;
  const int st = check_smla(shape);
  if (st) return st;
  if (!good_scale(softmax_scale)) return ATTN_ERR_RANGE;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(dout) || !aligned16(dq) || !aligned16(dkv_accum) ||
      !aligned4(indices) || !aligned4(lse) || !aligned4(delta))
    return ATTN_ERR_ALIGN;
  return hip_status(launch_smla_bwd(q, kv, dout, indices, lse, delta, dq, dkv_accum, shape.tokens, shape.kv_tokens,
                                    shape.heads, shape.topk, softmax_scale, (hipStream_t)stream));
}

size_t attn_sparse_mla_bwd_split_workspace_bytes(smla_shape shape) {
  if (check_smla(shape)) return 0;
  return smla_split_workspace_bytes(shape.tokens, shape.kv_tokens, shape.heads, shape.topk);
}

int attn_sparse_mla_bwd_split(const uint16_t* q, const uint16_t* kv, const uint16_t* dout, const int32_t* indices,
                              const float* lse, const float* delta, uint16_t* dq, uint16_t* dkv, void* workspace,
                              size_t workspace_bytes, smla_shape shape, float softmax_scale, void* stream) {
  if (!q || !kv || !dout || !indices || !lse || !delta || !dq || !dkv) return ATTN_ERR_NULL_PTR;
  const int st = check_smla(shape);
  if (st) return st;
  if (!good_scale(softmax_scale)) return ATTN_ERR_RANGE;
  if (!workspace ||
      workspace_bytes < smla_split_workspace_bytes(shape.tokens, shape.kv_tokens, shape.heads, shape.topk))
    return ATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(dout) || !aligned16(dq) || !aligned16(dkv) ||
      !aligned16(workspace) || !aligned4(indices) || !aligned4(lse) || !aligned4(delta))
    return ATTN_ERR_ALIGN;
  return hip_status(launch_smla_bwd_split(q, kv, dout, indices, lse, delta, dq, dkv, workspace, shape.tokens,
                                          shape.kv_tokens, shape.heads, shape.topk, softmax_scale,
                                          (hipStream_t)stream));
}

int attn_sparse_mla_bwd_postprocess(const float* dkv_accum, uint16_t* dkv, smla_shape shape, void* stream) {
  if (!dkv_accum || !dkv) return ATTN_ERR_NULL_PTR;
  const int st = check_smla(shape);
  if (st) return st;
  if (!aligned16(dkv_accum) || !aligned16(dkv)) return ATTN_ERR_ALIGN;
  return hip_status(launch_smla_bwd_post(dkv_accum, dkv, shape.kv_tokens, (hipStream_t)stream));
}

}  // extern "C"
