// Launchers of the sparse MLA backward's deterministic dKV path (host side,
// called by the C ABI).  Shapes and layouts as the other sparse MLA calls:
// q [T][H][576], kv [Tk][576], idx [T][K] int32, dout [T][H][512] bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mi355 {

// The backward kernel with dKV rows stored per entry: row pos[t*K + i] * n_ht
// + head tile of `part` ([T*K*n_ht + 1][576] fp32, the last row a sink for
// unused entries), n_ht = ceil(H / 32).
hipError_t launch_smla_bwd_partial(const uint16_t* q, const uint16_t* kv, const uint16_t* dout, const int* idx,
                                   const float* lse, const float* delta, uint16_t* dq, float* part, const int* pos,
                                   int T, int Tk, int H, int K, float scale, hipStream_t stream);

// Bytes of the workspace launch_smla_bwd_split carves up (partial rows,
// entry positions, key-row offsets, sort buffers and digit counts).
size_t smla_split_workspace_bytes(int T, int Tk, int H, int K);

// dq (bf16, written) and dkv = bf16 of a fixed-order sum of the per-entry
// partial rows (written whole, [Tk][576]).
hipError_t launch_smla_bwd_split(const uint16_t* q, const uint16_t* kv, const uint16_t* dout, const int* idx,
                                 const float* lse, const float* delta, uint16_t* dq, uint16_t* dkv, void* workspace,
                                 int T, int Tk, int H, int K, float scale, hipStream_t stream);

}  // namespace mi355
