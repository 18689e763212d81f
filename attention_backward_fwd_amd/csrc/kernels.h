// Launchers of the gfx950 attention kernels (host side, called by the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mi355 {

// Key-block height of the backward kernel for head dim D: 32-key tiles, one
// per wave of its 8 waves at D = 128 and two at D = 64 (whose dK/dV
// accumulators take half the registers).  The split dQ path keeps one fp32
// dQ partial per block of this many keys.
__host__ __device__ constexpr int bwd_block_n(int D) { return D == 64 ? 512 : 256; }

// Grouped-query attention: the number P of fp32 dK/dV partials the backward
// leaves per (key row, KV head).  One workgroup sweeps the query blocks of
// G / P query heads of a group one head after the other, so their dK/dV
// contributions add up in its accumulators and only P partials per group
// leave the kernel.  P is the smallest divisor of G that still gives the
// grid (B x Hkv x P x key blocks workgroups) two workgroups per CU; with
// fewer the causal key blocks, whose work differs up to n_blk-fold, would
// not even out over the CUs.
inline int bwd_gqa_parts(long long B, int Hkv, int G, int S, int D) {
  const long long blocks = B * Hkv * ((S + bwd_block_n(D) - 1) / bwd_block_n(D));
  for (int P = 1; P < G; P++)
    if (G % P == 0 && blocks * P >= 512) return P;
  return G;
}

// Packed variable-length sequences: when `cu` is set, "batch" b is sequence
// b of the packed rows: queries cu[b] .. cu[b+1]-1 of T query rows and keys
// cu_k[b] .. cu_k[b+1]-1 of Tk key rows (each range clamped to its tensor and
// cut to S, resp. Sk, rows: the bounds that size the grid), and the
// row-indexed tensors (LSE, Delta, dQ accumulator and partials) are
// head-major over all T query rows.  Otherwise sequence b is rows
// b*S .. b*S+S-1 of both (Sk == S, Tk unused).  Under causal masking query i
// of a sequence with lq queries and lk keys sees key j iff j <= i + lk - lq.
struct SeqRows {
  int base, len;  // first row and length of one sequence
};
__device__ __forceinline__ SeqRows seq_rows(const int* cu, int T, int b, int S) {
  if (!cu) return SeqRows{b * S, S};
  const int a = min(max(cu[b], 0), T);
  const int e = min(max(cu[b + 1], a), T);
  return SeqRows{a, min(e - a, S)};
}

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* cu;    // packed sequences: query offsets, or nullptr
  const int* cu_k;  // packed sequences: key offsets
  int T, Tk;        // query / key rows of the packed tensors (with cu)
  int B, S, Sk, Hq, G, Hkv, D;
  float scale;
  int causal;
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  const float* delta;
  float* dq_accum;  // fp32 atomic target (use_atomic) / sum output (split)
  float* dq_part;   // split path: [n_kv_blocks][B][S][Hq][D] fp32
  uint16_t* dk;     // groups == 1 outputs, [B][S][Hkv][D] bf16
  uint16_t* dv;
  float* dk_part;   // groups > 1: fp32 partials, [B][Sk][Hkv][G / hpw][D]
  float* dv_part;
  int hpw;          // query heads of a group per workgroup (divides G)
  const int* cu;    // packed sequences: query offsets, or nullptr
  const int* cu_k;  // packed sequences: key offsets
  int T, Tk;        // query / key rows of the packed tensors (with cu)
  int B, S, Sk, Hq, G, Hkv, D;
  float scale;
  float log2_scale;  // log2(scale), computed on the host
  int causal, use_atomic;
};

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);
hipError_t launch_preprocess(const uint16_t* o, const uint16_t* dout, float* delta, float* dq_accum,
                             int B, int S, int Hq, int D, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);
hipError_t launch_dq_sum(const float* dq_part, float* dq_accum, int B, int S, int Hq, int D,
                         int causal, hipStream_t stream);
// Packed sequences: rows of dq_accum are [Hq][T]; sums the key blocks each
// row sees of its own sequence, writes 0 to rows outside every sequence and
// to rows that see no key.
hipError_t launch_dq_sum_varlen(const float* dq_part, float* dq_accum, const int* cu, const int* cu_k, int n_seqs,
                                int T, int Tk, int S, int Sk, int Hq, int D, int causal, hipStream_t stream);
// Rows outside every sequence (capacity padding, and rows of a sequence past
// S) of up to two [T][heads][D] tensors (bf16, or fp32 when `fp32`) set to 0,
// and those rows of an [Hq][T] LSE set to lse_value; null tensors skipped.
hipError_t launch_pad_fill(void* x0, void* x1, int fp32, int heads, float* lse, int Hq, float lse_value,
                           const int* cu, int n_seqs, int T, int S, int D, hipStream_t stream);
// dq = bf16(dq_accum) over B*S query rows; with partials (dk_part set):
// dk/dv[row, kv] = bf16(sum of the P partials [row][kv][0 .. P-1]) over
// kv_rows key rows of Hkv heads.
hipError_t launch_postprocess(const float* dq_accum, const float* dk_part, const float* dv_part,
                              uint16_t* dq, uint16_t* dk, uint16_t* dv, int B, int S, int Hq, int Hkv, int P,
                              int D, long long kv_rows, hipStream_t stream);
hipError_t launch_gqa_reduce(const float* dk_part, const float* dv_part, uint16_t* dk, uint16_t* dv, int S, int Hq,
                             int Hkv, int P, int D, long long kv_rows, hipStream_t stream);

// Simple gated linear attention, chunked backward (head dim 128, chunks of
// 64): a forward sweep (state h, dq) and a backward sweep (state dH, dk, dv)
// in one launch, then the gate's reverse running sum.  Tensors
// [B][T][H][128] bf16, g and dg [B][T][H] fp32; the workspace holds the
// per-token q.dq and k.dk ([2][B*H][T] fp32).
hipError_t launch_gla_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                          const float* g, uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dg, void* workspace,
                          int B, int T, int H, float scale, hipStream_t stream);
size_t gla_bwd_workspace_bytes(int B, int T, int H);

// Largest kv_tokens of the sparse MLA calls (keeps every byte offset of the
// fp32 dKV accumulator below 2^31).
constexpr int kSmlaMaxKvTokens = 1 << 19;

// Sparse MLA (576-wide latent rows, 512 value channels) over per-token
// index lists: q [T][H][576], kv [Tk][576], idx [T][K] int32 (-1 or out of
// range: unused), o [T][H][512] bf16, lse [T][H] fp32.
hipError_t launch_smla_fwd(const uint16_t* q, const uint16_t* kv, const int* idx, uint16_t* o, float* lse, int T,
                           int Tk, int H, int K, float scale, hipStream_t stream);
// Backward: Delta [T][H] (and zeroing of the fp32 dKV accumulator [Tk][576]
// when given); dq [T][H][576] bf16 and atomic fp32 dKV; dkv = bf16(accumulator).
hipError_t launch_smla_bwd_pre(const uint16_t* o, const uint16_t* dout, float* delta, float* dkv_acc, int T, int Tk,
                               int H, hipStream_t stream);
hipError_t launch_smla_bwd(const uint16_t* q, const uint16_t* kv, const uint16_t* dout, const int* idx,
                           const float* lse, const float* delta, uint16_t* dq, float* dkv_acc, int T, int Tk, int H,
                           int K, float scale, hipStream_t stream);
hipError_t launch_smla_bwd_post(const float* dkv_acc, uint16_t* dkv, int Tk, hipStream_t stream);

hipError_t launch_merge(const uint16_t* o_parts, const float* lse_parts, int n_parts, uint16_t* o, float* lse,
                        int B, int S, int Hq, int D, hipStream_t stream);

}  // namespace mi355
