// Merge of partial attention results over disjoint key chunks, the step
// that context-parallel (ring) attention needs after each query chunk has
// met every key chunk it can see (see the context-parallel behaviour of the
// fused DSA path in Megatron-LM #5049):
//
//   LSE = log sum_k exp(LSE_k),     O = sum_k exp(LSE_k - LSE) O_k
//
// in fp32, with the forward kernel's convention for rows that see no key
// (LSE_k = -inf, O_k = 0): such parts carry weight 0, and a row empty in
// every part gets LSE = -inf and O = 0.  O is written as bf16 (RNE).
// HBM-bound: every part's O row and LSE are read once, 16 bytes per lane.
#include "common.h"
#include "kernels.h"

namespace mi355 {

namespace {

// One row (b, s, h) per D/8 lanes, 8 elements per lane; rows are numbered
// in the BSHD order of O, so that a wave's O accesses are one contiguous run
// (the [B][Hq][S] LSE values, 1/64 of the bytes, are gathered).
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const uint16_t* __restrict__ o_parts,
                                                    const float* __restrict__ lse_parts, int n_parts,
                                                    uint16_t* __restrict__ o, float* __restrict__ lse, int B,
                                                    int S, int Hq) {
  constexpr int TPR = D / 8;  // lanes per row
  const long long rows = (long long)B * Hq * S;
  const size_t part_elems = (size_t)rows * D;
  const int sub = threadIdx.x % TPR;
  const long long stride = (long long)gridDim.x * (256 / TPR);
  for (long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR; row < rows; row += stride) {
    const int h = (int)(row % Hq);
    const long long bs = row / Hq;
    const int s = (int)(bs % S), b = (int)(bs / S);
    const size_t off = (size_t)row * D + 8 * sub;                      // BSHD element offset
    const long long lrow = ((long long)b * Hq + h) * S + s;            // [B][Hq][S] index
    float m = -INFINITY;
    for (int k = 0; k < n_parts; k++) m = fmaxf(m, lse_parts[(size_t)k * rows + lrow]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float out_lse = -INFINITY;
    if (m != -INFINITY) {
      float z = 0.f;
      // Four parts per round, their O loads issued together.
      for (int k0 = 0; k0 < n_parts; k0 += 4) {
        u32x4 ov[4];
        float wk[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const int k = min(k0 + u, n_parts - 1);  // past the end: reread the last part, weight 0
          // Streaming load: each partial is read once.
          ov[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o_parts + (size_t)k * part_elems + off));
          wk[u] = k0 + u < n_parts ? __builtin_amdgcn_exp2f((lse_parts[(size_t)k * rows + lrow] - m) * kLog2e) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
          z += wk[u];
#pragma unroll
          for (int i = 0; i < 4; i++) {
            acc[2 * i] = fmaf(wk[u], __uint_as_float(ov[u][i] << 16), acc[2 * i]);
            acc[2 * i + 1] = fmaf(wk[u], __uint_as_float(ov[u][i] & 0xffff0000u), acc[2 * i + 1]);
          }
        }
      }
      const float inv = 1.f / z;
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] *= inv;
      out_lse = m + __builtin_amdgcn_logf(z) * kLn2;
    }
    *reinterpret_cast<u32x4*>(o + off) = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                              pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    if (sub == 0) lse[lrow] = out_lse;
  }
}

}  // namespace

hipError_t launch_merge(const uint16_t* o_parts, const float* lse_parts, int n_parts, uint16_t* o, float* lse,
                        int B, int S, int Hq, int D, hipStream_t stream) {
  const long long rows = (long long)B * Hq * S;
  const int per_block = 256 / (D / 8);
  long long g = (rows + per_block - 1) / per_block;
  if (g > 256LL * 64) g = 256LL * 64;
  if (g < 1) g = 1;
  if (D == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)g), dim3(256), 0, stream, o_parts, lse_parts, n_parts, o,
                       lse, B, S, Hq);
  else
    hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)g), dim3(256), 0, stream, o_parts, lse_parts, n_parts, o,
                       lse, B, S, Hq);
  return hipGetLastError();
}

}  // namespace mi355
