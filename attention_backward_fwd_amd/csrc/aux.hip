// Bandwidth-bound steps around the attention backward on gfx950:
//   preprocess   Delta = rowsum(dO o O) (+ zero the fp32 dQ accumulator)
//   dq_sum       split path: dQ = sum of the per-key-block partials, in
//                ascending block order
//   postprocess  dQ fp32 -> bf16 (head-major accumulator to BSHD);
//                grouped-query dK/dV partial reduction
// These are the flashattn_bwd_preprocess / flashattn_bwd_postprocess steps of
// the TileLang #940 examples and the "sum" half of its split+sum template.
// All moves are 16-byte vector loads/stores along contiguous rows.
#include "common.h"
#include "kernels.h"

namespace mi355 {

namespace {

// One row (b, s, h) per D/8 lanes, 8 elements per lane.  Rows are numbered
// (b, h, s) with s fastest so that Delta, stored [B][Hq][S], is written with
// consecutive addresses by neighbouring row groups.
template <int D>
__global__ __launch_bounds__(256) void preprocess_kernel(const uint16_t* __restrict__ o,
                                                         const uint16_t* __restrict__ dout,
                                                         float* __restrict__ delta,
                                                         float* __restrict__ dq_accum, int B, int S,
                                                         int Hq) {
  constexpr int TPR = D / 8;  // lanes per row
  const long long rows = (long long)B * Hq * S;
  const int sub = threadIdx.x % TPR;
  const long long stride = (long long)gridDim.x * (256 / TPR);
  for (long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR; row < rows; row += stride) {
    const int s = (int)(row % S);
    const long long bh = row / S;
    const int h = (int)(bh % Hq), b = (int)(bh / Hq);
    const size_t off = ((size_t)((long long)b * S + s) * Hq + h) * D + 8 * sub;
    const u32x4 ov = *reinterpret_cast<const u32x4*>(o + off);
    const u32x4 dv = *reinterpret_cast<const u32x4*>(dout + off);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      acc = fmaf(__uint_as_float(ov[i] << 16), __uint_as_float(dv[i] << 16), acc);
      acc = fmaf(__uint_as_float(ov[i] & 0xffff0000u), __uint_as_float(dv[i] & 0xffff0000u), acc);
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (sub == 0) delta[row] = acc;
    if (dq_accum) {  // head-major [B][Hq][S][D]: row `row` starts at row * D
      // Each store instruction covers whole lines (a row's first half, then
      // its second half: 16 bytes per lane, consecutive lanes adjacent), not
      // every other 16 bytes.  (Plain stores: streaming ones measured faster
      // only when the caches hold nothing dirty, and slower after other work.)
      f32x4* z = reinterpret_cast<f32x4*>(dq_accum + (size_t)row * D + 4 * sub);
      z[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      z[TPR] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// dq_accum[b,h,s,:] = sum_{j=0..J(s)} part[j][b,h,s,:], ascending j, where
// J(s) is the last key block (causal: the block holding key s).  Both are
// head-major fp32 [B][Hq][S][D].
// acc + part[0] + part[1] + ... + part[n-1] (16-byte slots `slot` floats
// apart), added one at a time in ascending order, so the bits do not depend on
// how the loads are grouped; the loads are issued up to eight at a time so
// that they are in flight together instead of one memory latency apart.
// fp32 partials written with streaming stores and read once: streaming
// loads keep them from displacing other data in the caches (17% faster for
// the split path's sum at 4 x 32 x 4096 x 128).
__device__ __forceinline__ f32x4 ld_stream(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

__device__ __forceinline__ f32x4 sum_slots(f32x4 acc, const float* part, size_t slot, int n) {
  auto ld = [&](int j) { return ld_stream(part + (size_t)j * slot); };
  int j = 0;
  for (; j + 16 <= n; j += 16) {
    f32x4 v[16];
#pragma unroll
    for (int u = 0; u < 16; u++) v[u] = ld(j + u);
#pragma unroll
    for (int u = 0; u < 16; u++) acc += v[u];
  }
  for (; j + 8 <= n; j += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; u++) v[u] = ld(j + u);
#pragma unroll
    for (int u = 0; u < 8; u++) acc += v[u];
  }
  if (j + 4 <= n) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) v[u] = ld(j + u);
#pragma unroll
    for (int u = 0; u < 4; u++) acc += v[u];
    j += 4;
  }
  for (; j < n; j++) acc += ld(j);
  return acc;
}

__global__ __launch_bounds__(256) void dq_sum_kernel(const float* __restrict__ part,
                                                     float* __restrict__ dq, long long n4, int S,
                                                     int D, int n_nblk, int bn, int causal) {
  const size_t slot = (size_t)n4 * 4;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) {
    const long long e = i * 4;
    const int s = (int)((e / D) % S);
    const int last = causal ? s / bn : n_nblk - 1;
    const float* src = part + e;
    const f32x4 acc = sum_slots(ld_stream(src), src + slot, slot, last);
    *reinterpret_cast<f32x4*>(dq + e) = acc;
  }
}

// Packed sequences: the sequence holding row t, found by bisection over the
// clamped sequence starts (non-decreasing when cu_seqlens is), with its first
// row and its length cut to S rows; -1 for rows outside every such range
// (capacity padding, or rows of a sequence past S).
__device__ __forceinline__ int seq_of_row(const int* cu, int n_seqs, int T, int S, int t, int& start, int& len) {
  if (n_seqs < 1) return -1;
  const int first = min(max(cu[0], 0), T);
  if (t < first || t >= min(max(cu[n_seqs], first), T)) return -1;
  int lo = 0, hi = n_seqs - 1;  // largest b with start_b <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (min(max(cu[mid], 0), T) <= t) lo = mid; else hi = mid - 1;
  }
  const SeqRows r = seq_rows(cu, T, lo, S);
  start = r.base;
  len = r.len;
  return t >= r.base && t < r.base + r.len ? lo : -1;
}

// Packed sequences, split path: dq_accum[h, t, :] = sum over the key blocks
// j = 0 .. J of row t's own sequence of part[j][h, t, :], in ascending j, J
// being the block of the last key the row sees (under causal masking, key
// position + lk - lq; else the sequence's last key); 0 for rows outside every
// sequence and rows that see no key.  Rows are [Hq][T].
__global__ __launch_bounds__(256) void dq_sum_varlen_kernel(const float* __restrict__ part,
                                                            float* __restrict__ dq, const int* __restrict__ cu,
                                                            const int* __restrict__ cu_k, int n_seqs, int T,
                                                            int Tk, int S, int Sk, long long n4, int D,
                                                            int bn, int causal) {
  const size_t slot = (size_t)n4 * 4;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) {
    const long long e = i * 4;
    const int t = (int)((e / D) % T);
    int start = 0, len = 0;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int b = seq_of_row(cu, n_seqs, T, S, t, start, len);
    if (b >= 0) {
      const int lk = seq_rows(cu_k, Tk, b, Sk).len;
      const int last_key = causal ? min(t - start + lk - len, lk - 1) : lk - 1;
      const float* src = part + e;
      if (last_key >= 0) acc = sum_slots(acc, src, slot, last_key / bn + 1);
    }
    *reinterpret_cast<f32x4*>(dq + e) = acc;
  }
}

// Rows of packed tensors outside every sequence (see seq_of_row): the rows of
// [T][heads][D] tensors x0 and x1 (bf16, or fp32 when `fp32`; either may be
// null) set to 0, and those rows of an [Hq][T] LSE (may be null) set to
// lse_value.  With non-decreasing offsets these rows are the ranges before
// the first sequence and after the last one, plus the tail of any sequence
// cut to S rows: workgroups 0 .. 2*kPadSplit-1 share the two outer ranges,
// workgroup 2*kPadSplit + b takes sequence b's cut tail (normally empty).
// Every range is clamped to [0, T].
constexpr int kPadSplit = 128;
__global__ __launch_bounds__(256) void pad_fill_kernel(void* __restrict__ x0, void* __restrict__ x1, int fp32,
                                                       int heads, float* __restrict__ lse, int Hq, float lse_value,
                                                       const int* __restrict__ cu, int n_seqs, int T, int S, int D) {
  const int per_row = heads * D / (fp32 ? 4 : 8);  // 16-byte chunks per row
  const int first = min(max(cu[0], 0), T);
  int lo, hi, r0, step;
  if ((int)blockIdx.x < 2 * kPadSplit) {
    const bool tail = blockIdx.x >= kPadSplit;
    lo = tail ? (n_seqs > 0 ? min(max(cu[n_seqs], first), T) : first) : 0;
    hi = tail ? T : first;
    r0 = blockIdx.x % kPadSplit;
    step = kPadSplit;
  } else {
    const int b = blockIdx.x - 2 * kPadSplit;
    const SeqRows r = seq_rows(cu, T, b, S);
    lo = r.base + r.len;
    hi = min(max(cu[b + 1], r.base), T);
    r0 = 0;
    step = 1;
  }
  for (int t = lo + r0; t < hi; t += step) {
    const size_t row = (size_t)t * per_row;
    for (int c = threadIdx.x; c < per_row; c += 256) {
      if (x0) reinterpret_cast<u32x4*>(x0)[row + c] = u32x4{0u, 0u, 0u, 0u};
      if (x1) reinterpret_cast<u32x4*>(x1)[row + c] = u32x4{0u, 0u, 0u, 0u};
    }
    if (lse)
      for (int h = threadIdx.x; h < Hq; h += 256) lse[(size_t)h * T + t] = lse_value;
  }
}

__device__ __forceinline__ u32x2 cvt4(f32x4 a) { return u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])}; }

// Part 1 (chunks [0, nq8)): dq[b,s,h,:] = bf16(dq_accum[b,h,s,:]), 8 elements
// per chunk (chunks numbered in the BSHD output order; chunk c of a row takes
// elements 4c.. of each half of the row).
// Part 2 (chunks [nq8, nq8 + nkv8), grouped queries only): dk/dv chunk of
// (b, s, kv) = bf16(sum_r partial[b, s, kv, r]), ascending r < G (here G is
// the number of partials per key row and KV head).
__global__ __launch_bounds__(256) void postprocess_kernel(const float* __restrict__ dq_accum,
                                                          const float* __restrict__ dk_part,
                                                          const float* __restrict__ dv_part,
                                                          uint16_t* __restrict__ dq, uint16_t* __restrict__ dk,
                                                          uint16_t* __restrict__ dv, long long nq8,
                                                          long long nkv8, int G, int D, int S, int Hq) {
  const long long total = nq8 + nkv8;
  const int dchunks = D / 8;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    if (i < nq8) {
      const long long row = i / dchunks;  // (b, s, h) of the output
      const int d0 = (int)(i % dchunks) * 8;
      const int h = (int)(row % Hq);
      const long long bs = row / Hq;
      const int s = (int)(bs % S);
      const long long b = bs / S;
      // Plain loads: the accumulator was just written (atomics, or the
      // split path's sum) and is usually still in the last-level cache.
      // Chunk c of a row takes elements 4c.. of each half of the row, so
      // that each load and store instruction covers whole lines.
      const int c4 = d0 / 2;
      const float* src = dq_accum + ((b * Hq + h) * S + s) * D + c4;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 a2 = *reinterpret_cast<const f32x4*>(src + D / 2);
      uint16_t* dst = dq + row * D + c4;
      *reinterpret_cast<u32x2*>(dst) = cvt4(a);
      *reinterpret_cast<u32x2*>(dst + D / 2) = cvt4(a2);
    } else {
      const long long c = i - nq8;          // chunk of the [B,S,Hkv,D] output
      const long long rowkv = c / dchunks;  // (b, s, kv) flattened
      const int d0 = (int)(c % dchunks) * 8;
      const int c4 = d0 / 2;  // elements 4c.. of each half of the row, as for dQ
      const size_t base = (size_t)rowkv * G * D + c4;  // partial row (b, s, kv, 0)
      f32x4 k0 = {0, 0, 0, 0}, k1 = {0, 0, 0, 0}, v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
      for (int r = 0; r < G; r++) {
        const float* pk = dk_part + base + (size_t)r * D;
        const float* pv = dv_part + base + (size_t)r * D;
        k0 += ld_stream(pk);
        k1 += ld_stream(pk + D / 2);
        v0 += ld_stream(pv);
        v1 += ld_stream(pv + D / 2);
      }
      uint16_t* dkr = dk + rowkv * D + c4;
      uint16_t* dvr = dv + rowkv * D + c4;
      *reinterpret_cast<u32x2*>(dkr) = cvt4(k0);
      *reinterpret_cast<u32x2*>(dkr + D / 2) = cvt4(k1);
      *reinterpret_cast<u32x2*>(dvr) = cvt4(v0);
      *reinterpret_cast<u32x2*>(dvr + D / 2) = cvt4(v1);
    }
  }
}

unsigned grid_for(long long work, long long per_block) {
  long long g = (work + per_block - 1) / per_block;
  // One work item per thread (the kernels still loop, for grids past the
  // cap): every thread's loads are in flight at once.
  const long long cap = 1LL << 30;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_preprocess(const uint16_t* o, const uint16_t* dout, float* delta, float* dq_accum,
                             int B, int S, int Hq, int D, hipStream_t stream) {
  const long long rows = (long long)B * Hq * S;
  if (D == 64)
    hipLaunchKernelGGL(preprocess_kernel<64>, dim3(grid_for(rows, 32)), dim3(256), 0, stream, o, dout, delta,
                       dq_accum, B, S, Hq);
  else
    hipLaunchKernelGGL(preprocess_kernel<128>, dim3(grid_for(rows, 16)), dim3(256), 0, stream, o, dout, delta,
                       dq_accum, B, S, Hq);
  return hipGetLastError();
}

hipError_t launch_dq_sum(const float* dq_part, float* dq_accum, int B, int S, int Hq, int D, int causal,
                         hipStream_t stream) {
  const long long n4 = (long long)B * S * Hq * D / 4;
  const int bn = bwd_block_n(D), n_nblk = (S + bn - 1) / bn;
  // One element group per thread (no grid-stride loop): every thread's slot
  // loads are in flight at once.
  hipLaunchKernelGGL(dq_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, dq_part, dq_accum, n4, S, D,
                     n_nblk, bn, causal);
  return hipGetLastError();
}

hipError_t launch_dq_sum_varlen(const float* dq_part, float* dq_accum, const int* cu, const int* cu_k, int n_seqs,
                                int T, int Tk, int S, int Sk, int Hq, int D, int causal, hipStream_t stream) {
  const long long n4 = (long long)T * Hq * D / 4;
  hipLaunchKernelGGL(dq_sum_varlen_kernel, dim3(grid_for(n4, 256)), dim3(256), 0, stream, dq_part, dq_accum, cu,
                     cu_k, n_seqs, T, Tk, S, Sk, n4, D, bwd_block_n(D), causal);
  return hipGetLastError();
}

hipError_t launch_pad_fill(void* x0, void* x1, int fp32, int heads, float* lse, int Hq, float lse_value,
                           const int* cu, int n_seqs, int T, int S, int D, hipStream_t stream) {
  hipLaunchKernelGGL(pad_fill_kernel, dim3(2 * kPadSplit + n_seqs), dim3(256), 0, stream, x0, x1, fp32, heads, lse,
                     Hq, lse_value, cu, n_seqs, T, S, D);
  return hipGetLastError();
}

hipError_t launch_postprocess(const float* dq_accum, const float* dk_part, const float* dv_part, uint16_t* dq,
                              uint16_t* dk, uint16_t* dv, int B, int S, int Hq, int Hkv, int P, int D,
                              long long kv_rows, hipStream_t stream) {
  const long long nq8 = (long long)B * S * Hq * D / 8;
  const long long nkv8 = dk_part ? kv_rows * Hkv * D / 8 : 0;
  hipLaunchKernelGGL(postprocess_kernel, dim3(grid_for(nq8 + nkv8, 256)), dim3(256), 0, stream, dq_accum,
                     dk_part, dv_part, dq, dk, dv, nq8, nkv8, P, D, S, Hq);
  return hipGetLastError();
}

// The dK/dV half of the postprocess alone: dk/dv[b,s,kv,:] = bf16(sum over
// r < P, ascending, of the partials).
hipError_t launch_gqa_reduce(const float* dk_part, const float* dv_part, uint16_t* dk, uint16_t* dv, int S, int Hq,
                             int Hkv, int P, int D, long long kv_rows, hipStream_t stream) {
  const long long nkv8 = kv_rows * Hkv * D / 8;
  hipLaunchKernelGGL(postprocess_kernel, dim3(grid_for(nkv8, 256)), dim3(256), 0, stream, nullptr, dk_part,
                     dv_part, nullptr, dk, dv, 0LL, nkv8, P, D, S, Hq);
  return hipGetLastError();
}

}  // namespace mi355
