// Launchers of the gfx950 attention kernels (host side, called by the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mi355 {

// Key-block height of the backward kernel; the split dQ path keeps one fp32
// dQ partial per block of this many keys.
constexpr int kBwdBlockN = 256;

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, S, Hq, G, Hkv, D;
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
  float* dk_part;   // groups > 1: per-query-head partials, [B][S][Hq][D] fp32
  float* dv_part;
  int B, S, Hq, G, Hkv, D;
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
hipError_t launch_postprocess(const float* dq_accum, const float* dk_part, const float* dv_part,
                              uint16_t* dq, uint16_t* dk, uint16_t* dv, int B, int S, int Hq, int G,
                              int D, hipStream_t stream);

hipError_t launch_merge(const uint16_t* o_parts, const float* lse_parts, int n_parts, uint16_t* o, float* lse,
                        int B, int S, int Hq, int D, hipStream_t stream);

}  // namespace mi355
