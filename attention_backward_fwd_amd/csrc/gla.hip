// Chunked backward of simple gated linear attention (one scalar log-decay per
// token and head), the first of the chunk backward kernels that the
// flash-linear-attention pull request "[Perf] TileLang backends for
// linear-attention chunk backward (simple_gla / gla / delta_rule / gdn)"
// (fla-org/flash-linear-attention #1046, summary) speeds up: a chunk state
// recurrence and a per-chunk dq/dk/dv/dg stage.
//
// Definition (per batch b and head h; G the running sum of g):
//   o_t  = scale * sum_{s<=t} exp(G_t - G_s) (q_t . k_s) v_s
//   dq_t = scale * sum_{s<=t} exp(G_t - G_s) (do_t . v_s) k_s
//   dk_s = scale * sum_{t>=s} exp(G_t - G_s) (do_t . v_s) q_t
//   dv_s = scale * sum_{t>=s} exp(G_t - G_s) (q_t . k_s) do_t
//   dg_r = sum_{t>=r} (q_t . dq_t - k_t . dk_t)
// Chunks of C = 64 tokens, G taken inside each chunk (exp never exceeds 1
// for g <= 0).  With h_n the state entering chunk n and dH_n the gradient of
// h_n:
//   h_{n+1}  = exp(Gl) h_n + sum_s exp(Gl - G_s) k_s^T v_s
//   dH_n     = exp(Gl) dH_{n+1} + scale sum_t exp(G_t) q_t^T do_t
//   dq_t     = scale [sum_{s<=t} e^{G_t-G_s}(do_t.v_s) k_s + e^{G_t} do_t h_n^T]
//   dk_s     = scale sum_{t>=s} e^{G_t-G_s}(do_t.v_s) q_t + e^{Gl-G_s} v_s dH_{n+1}^T
//   dv_s     = scale sum_{t>=s} e^{G_t-G_s}(q_t.k_s) do_t + e^{Gl-G_s} k_s dH_{n+1}
// (Gl: G at the chunk's last token).  Kernels: gla_states (h_n forward and
// dH_{n+1} backward, bf16 to the workspace), gla_dqkv (one chunk per
// workgroup: dq, dk, dv and the per-token q.dq - k.dk), gla_dg (reverse
// running sum over the sequence).
#include "common.h"
#include "kernels.h"

namespace mi355 {

namespace {

constexpr int kC = 64;   // chunk length
constexpr int kD = 128;  // head dim (K = V)

// 32x32x16 operands from swizzled LDS tiles of DT-wide rows.  Both readers
// hand out the k index of each 16-step in the same order (lane half hi gets
// k = 4hi .. 4hi+3 and 8+4hi .. 8+4hi+3, the order of the rows of a 32x32
// result's elements 0..7), so any pairing of them multiplies matching k.
//   op_row: tile stored [x][k] (x = the lane's m or n index)
//   op_tr:  tile stored [k][x]
template <int DT>
__device__ __forceinline__ bf16x8 op_row(const uint16_t* t, int x0, int k0, int lane) {
  const int r = x0 + (lane & 31), hi = lane >> 5;
  const u32x2 a = *reinterpret_cast<const u32x2*>(t + swz_off<DT>(r, k0 + 4 * hi));
  const u32x2 b = *reinterpret_cast<const u32x2*>(t + swz_off<DT>(r, k0 + 8 + 4 * hi));
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}
template <int DT>
__device__ __forceinline__ bf16x8 op_tr(const uint16_t* t, int k0, int x0, int lane) {
  const int hi = lane >> 5, L = lane & 15, gp = (lane >> 4) & 1;
  const int col = x0 + 16 * gp + 4 * (L & 3);
  return lds_read_tr8(t + swz_off<DT>(k0 + 4 * hi + (L >> 2), col), t + swz_off<DT>(k0 + 8 + 4 * hi + (L >> 2), col));
}
// The k index (0..15 within a 16-step) of element i of a lane's operand.
__device__ __forceinline__ int op_k(int i, int hi) { return (i < 4 ? 4 * hi + i : 8 + 4 * hi + (i - 4)); }

// Row of element j of a 32x32 result held by a lane of half hi.
__device__ __forceinline__ int c_row(int j, int hi) { return 8 * (j >> 2) + 4 * hi + (j & 3); }

// Chunk-local inclusive running sum of g over the chunk's valid rows (rows
// past nv count 0), into sG[0..63]; one wave.  Returns nothing; callers
// barrier before reading.
__device__ __forceinline__ void chunk_cumsum(const float* g, size_t stride, int nv, float* sG, int lane) {
  float x = lane < nv ? g[(size_t)lane * stride] : 0.f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  sG[lane] = x;
}

// Scale the 8 values of an operand by per-k factors f[k0 + op_k(i)].
__device__ __forceinline__ bf16x8 scale_op(bf16x8 v, const float* f, int k0, int hi) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; i++) x[i] = (float)v[i] * f[k0 + op_k(i, hi)];
  return pack8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
}

// ------------------------------------------------------------ chunk states
// Workgroup (b*H + h, vt, dir): 4 waves own the 128 x 64 state tile of value
// columns 64vt .. 64vt+63 (wave w: rows 32w .. 32w+31, two 32x32 tiles).
// dir 0 sweeps chunks forward and writes h_n (the state entering chunk n);
// dir 1 sweeps backward and writes dH_{n+1} (zero for the last chunk).
// Per chunk: X (k or q) and Y (v or do) tiles arrive by LDS-DMA one chunk
// ahead; the update is S = exp(Gl) S + X^T (f o Y) with
// f_s = exp(Gl - G_s) (forward) or scale * exp(G_t) (backward), 0 past the
// end of the sequence.
__global__ __launch_bounds__(256) void gla_states_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const uint16_t* __restrict__ dout,
                                                         const float* __restrict__ g, uint16_t* __restrict__ hs,
                                                         uint16_t* __restrict__ dhs, int T, int H, float scale) {
  __shared__ __attribute__((aligned(16))) uint16_t sX0[kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sX1[kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sY0[kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sY1[kC * kD];
  __shared__ float sG[kC];
  __shared__ float sF[kC];

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), hi = lane >> 5;
  const int bh = blockIdx.x, vt = blockIdx.y, dir = blockIdx.z;
  const int b = bh / H, h = bh % H;
  const int N = (T + kC - 1) / kC;
  const size_t rs = (size_t)H * kD;
  const uint16_t* X = (dir ? q : k) + ((size_t)b * T * H + h) * kD;
  const uint16_t* Y = (dir ? dout : v) + ((size_t)b * T * H + h) * kD;
  const float* gb = g + (size_t)b * T * H + h;
  uint16_t* out = (dir ? dhs : hs) + (size_t)bh * N * kD * kD;

  f32x16 acc[2] = {f32x16{}, f32x16{}};
  auto load = [&](int n, uint16_t* sx, uint16_t* sy) {
    tile_load_async<kD, kC, 4>(X, rs, n * kC, T, sx, w, lane);
    tile_load_async<kD, kC, 4>(Y, rs, n * kC, T, sy, w, lane);
  };
  auto store = [&](int n) {  // the state tile as bf16, rows 32w.., cols 64vt + 32nb + l32
    uint16_t* o = out + (size_t)n * kD * kD;
#pragma unroll
    for (int nb = 0; nb < 2; nb++)
#pragma unroll
      for (int j = 0; j < 16; j++)
        o[(size_t)(32 * w + c_row(j, hi)) * kD + 64 * vt + 32 * nb + (lane & 31)] = to_bf16(acc[nb][j]);
  };
  auto chunk = [&](int n, const uint16_t* sx, const uint16_t* sy) {
    const int nv = min(kC, T - n * kC);
    if (w == 0) chunk_cumsum(gb + (size_t)n * kC * H, H, nv, sG, lane);
    lds_barrier();
    const float gl = sG[nv - 1];
    if (w == 0) {
      const float f = dir ? scale * __expf(sG[lane]) : __expf(gl - sG[lane]);
      sF[lane] = lane < nv ? f : 0.f;
    }
    lds_barrier();
    const float decay = __expf(gl);
#pragma unroll
    for (int nb = 0; nb < 2; nb++) acc[nb] *= decay;
#pragma unroll
    for (int ks = 0; ks < kC / 16; ks++) {
      const bf16x8 a = op_tr<kD>(sx, 16 * ks, 32 * w, lane);
#pragma unroll
      for (int nb = 0; nb < 2; nb++) {
        const bf16x8 bb = scale_op(op_tr<kD>(sy, 16 * ks, 64 * vt + 32 * nb, lane), sF, 16 * ks, hi);
        acc[nb] = mfma32(a, bb, acc[nb]);
      }
    }
  };

  // Forward: chunks 0, 1, ..., storing the state before each update.
  // Backward: chunks N-1, ..., 0, storing dH_{n+1} before the update.
  const int first = dir ? N - 1 : 0, stepn = dir ? -1 : 1;
  load(first, sX0, sY0);
  for (int i = 0; i < N; i += 2) {
    const int n0 = first + stepn * i;
    store(n0);
    wait_vmem();
    lds_barrier();  // chunk n0 resident in buffer 0; buffer 1 free
    if (i + 1 < N) load(n0 + stepn, sX1, sY1);
    chunk(n0, sX0, sY0);
    if (i + 1 < N) {
      const int n1 = n0 + stepn;
      store(n1);
      wait_vmem();
      lds_barrier();
      if (i + 2 < N) load(n1 + stepn, sX0, sY0);
      chunk(n1, sX1, sY1);
    }
  }
}

// ------------------------------------------------------------ per-chunk stage
// Workgroup (chunk n, b*H + h), 4 waves.  LDS: q, k, v, do of the chunk
// [64][128], h_n and dH_{n+1} [128][128] (bf16, from the states kernel),
// the masked score matrices Mqk[t][s] = scale e^{G_t - G_s} (q_t.k_s) and
// Mdov[t][s] = scale e^{G_t - G_s} (do_t.v_s) for s <= t < nv (0 elsewhere).
// Outputs: dq, dk, dv (bf16) of the chunk's valid rows and
// dG_t = q_t.dq_t - k_t.dk_t (fp32), summed over the sequence by gla_dg.
__global__ __launch_bounds__(256) void gla_dqkv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ g, const uint16_t* __restrict__ hs,
                                                       const uint16_t* __restrict__ dhs, uint16_t* __restrict__ dq,
                                                       uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                                                       float* __restrict__ dG, int T, int H, float scale) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sK[kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sO[kC * kD];  // dO
  __shared__ __attribute__((aligned(16))) uint16_t sH[kD * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sDH[kD * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sMqk[kC * kC];
  __shared__ __attribute__((aligned(16))) uint16_t sMdov[kC * kC];
  __shared__ float sG[kC];
  __shared__ float sdG[2][2][kC];  // [q.dq or k.dk][column half][row], each entry written once

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), hi = lane >> 5;
  const int l32 = lane & 31;
  const int n = blockIdx.x, bh = blockIdx.y;
  const int b = bh / H, h = bh % H;
  const int N = (T + kC - 1) / kC;
  const int nv = min(kC, T - n * kC);
  const size_t rs = (size_t)H * kD;
  const size_t base = ((size_t)b * T * H + h) * kD;
  const size_t st_off = ((size_t)bh * N + n) * kD * kD;

  tile_load_async<kD, kC, 4>(q + base, rs, n * kC, T, sQ, w, lane);
  tile_load_async<kD, kC, 4>(k + base, rs, n * kC, T, sK, w, lane);
  tile_load_async<kD, kC, 4>(v + base, rs, n * kC, T, sV, w, lane);
  tile_load_async<kD, kC, 4>(dout + base, rs, n * kC, T, sO, w, lane);
  tile_load_async<kD, kD, 4>(hs + st_off, kD, 0, kD, sH, w, lane);
  tile_load_async<kD, kD, 4>(dhs + st_off, kD, 0, kD, sDH, w, lane);
  if (w == 1) chunk_cumsum(g + (size_t)b * T * H + h + (size_t)n * kC * H, H, nv, sG, lane);
  wait_vmem();
  lds_barrier();

  // Masked score matrices: wave w computes the 32x32 block (s-block w >> 1,
  // t-block w & 1) of both, as S^T[s][t] (A = k or v rows, B = q or do rows),
  // and writes them transposed, [t][s], four s values per 8-byte store.
  {
    const int sb = w >> 1, tb = w & 1;
    f32x16 a_qk = f32x16{}, a_dov = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kD / 16; ks++) {
      a_qk = mfma32(op_row<kD>(sK, 32 * sb, 16 * ks, lane), op_row<kD>(sQ, 32 * tb, 16 * ks, lane), a_qk);
      a_dov = mfma32(op_row<kD>(sV, 32 * sb, 16 * ks, lane), op_row<kD>(sO, 32 * tb, 16 * ks, lane), a_dov);
    }
    const int t = 32 * tb + l32;
    const float gt = sG[t];
#pragma unroll
    for (int jg = 0; jg < 4; jg++) {
      float mq[4], md[4];
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int s = 32 * sb + c_row(4 * jg + jj, hi);
        const float f = (s <= t && t < nv) ? scale * __expf(gt - sG[s]) : 0.f;
        mq[jj] = a_qk[4 * jg + jj] * f;
        md[jj] = a_dov[4 * jg + jj] * f;
      }
      const int s0 = 32 * sb + c_row(4 * jg, hi);
      *reinterpret_cast<u32x2*>(sMqk + swz_off<kC>(t, s0)) = u32x2{pack_bf16x2(mq[0], mq[1]), pack_bf16x2(mq[2], mq[3])};
      *reinterpret_cast<u32x2*>(sMdov + swz_off<kC>(t, s0)) = u32x2{pack_bf16x2(md[0], md[1]), pack_bf16x2(md[2], md[3])};
    }
  }
  lds_barrier();

  // Output tiles: wave w owns rows 32(w & 1) .. (t or s) and columns
  // 64(w >> 1) .. +63 (two 32x32 tiles) of each of dq, dk, dv.
  const int rb = w & 1, cb = w >> 1;
  const size_t orow = base + (size_t)n * kC * rs;  // element offset of the chunk's first row
  auto emit = [&](uint16_t* dst, const f32x16* x) {
#pragma unroll
    for (int nb = 0; nb < 2; nb++)
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int r = 32 * rb + c_row(j, hi);
        if (r < nv) dst[orow + (size_t)r * rs + 64 * cb + 32 * nb + l32] = to_bf16(x[nb][j]);
      }
  };
  // Row sums of x o src over this wave's 64 columns, into sdG[kind][cb]
  // (fixed-order sums: no atomics, so dG is reproducible bit for bit).
  auto dg_part = [&](const f32x16* x, const uint16_t* src, int kind) {
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int r = 32 * rb + c_row(j, hi);
      float p = 0.f;
#pragma unroll
      for (int nb = 0; nb < 2; nb++) p += x[nb][j] * from_bf16(src[swz_off<kD>(r, 64 * cb + 32 * nb + (l32 & ~3)) + (l32 & 3)]);
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) p += __shfl_xor(p, o, 64);
      if (l32 == 0) sdG[kind][cb][r] = p;
    }
  };

  // dq = Mdov k + scale e^{G_t} do h^T
  {
    f32x16 a1[2] = {f32x16{}, f32x16{}}, a2[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < kC / 16; ks++) {
      const bf16x8 am = op_row<kC>(sMdov, 32 * rb, 16 * ks, lane);
#pragma unroll
      for (int nb = 0; nb < 2; nb++) a1[nb] = mfma32(am, op_tr<kD>(sK, 16 * ks, 64 * cb + 32 * nb, lane), a1[nb]);
    }
#pragma unroll
    for (int ks = 0; ks < kD / 16; ks++) {
      const bf16x8 ao = op_row<kD>(sO, 32 * rb, 16 * ks, lane);
#pragma unroll
      for (int nb = 0; nb < 2; nb++) a2[nb] = mfma32(ao, op_row<kD>(sH, 64 * cb + 32 * nb, 16 * ks, lane), a2[nb]);
    }
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const float f = scale * __expf(sG[32 * rb + c_row(j, hi)]);
#pragma unroll
      for (int nb = 0; nb < 2; nb++) a1[nb][j] += f * a2[nb][j];
    }
    emit(dq, a1);
    dg_part(a1, sQ, 0);
  }
  const float gl = sG[nv - 1];
  // dk = Mdov^T q + e^{Gl - G_s} v dH^T
  {
    f32x16 a1[2] = {f32x16{}, f32x16{}}, a2[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < kC / 16; ks++) {
      const bf16x8 am = op_tr<kC>(sMdov, 16 * ks, 32 * rb, lane);
#pragma unroll
      for (int nb = 0; nb < 2; nb++) a1[nb] = mfma32(am, op_tr<kD>(sQ, 16 * ks, 64 * cb + 32 * nb, lane), a1[nb]);
    }
#pragma unroll
    for (int ks = 0; ks < kD / 16; ks++) {
      const bf16x8 av = op_row<kD>(sV, 32 * rb, 16 * ks, lane);
#pragma unroll
      for (int nb = 0; nb < 2; nb++) a2[nb] = mfma32(av, op_row<kD>(sDH, 64 * cb + 32 * nb, 16 * ks, lane), a2[nb]);
    }
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const float f = __expf(gl - sG[32 * rb + c_row(j, hi)]);
#pragma unroll
      for (int nb = 0; nb < 2; nb++) a1[nb][j] += f * a2[nb][j];
    }
    emit(dk, a1);
    dg_part(a1, sK, 1);
  }
  // dv = Mqk^T do + e^{Gl - G_s} k dH
  {
    f32x16 a1[2] = {f32x16{}, f32x16{}}, a2[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < kC / 16; ks++) {
      const bf16x8 am = op_tr<kC>(sMqk, 16 * ks, 32 * rb, lane);
#pragma unroll
      for (int nb = 0; nb < 2; nb++) a1[nb] = mfma32(am, op_tr<kD>(sO, 16 * ks, 64 * cb + 32 * nb, lane), a1[nb]);
    }
#pragma unroll
    for (int ks = 0; ks < kD / 16; ks++) {
      const bf16x8 ak = op_row<kD>(sK, 32 * rb, 16 * ks, lane);
#pragma unroll
      for (int nb = 0; nb < 2; nb++) a2[nb] = mfma32(ak, op_tr<kD>(sDH, 16 * ks, 64 * cb + 32 * nb, lane), a2[nb]);
    }
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const float f = __expf(gl - sG[32 * rb + c_row(j, hi)]);
#pragma unroll
      for (int nb = 0; nb < 2; nb++) a1[nb][j] += f * a2[nb][j];
    }
    emit(dv, a1);
  }
  lds_barrier();
  if (w == 0 && lane < nv)
    dG[(size_t)b * T * H + (size_t)(n * kC + lane) * H + h] =
        (sdG[0][0][lane] + sdG[0][1][lane]) - (sdG[1][0][lane] + sdG[1][1][lane]);
}

// dg[b, t, h] = sum_{t' >= t} dG[b, t', h]: one wave per (b, h), 64 tokens
// per step from the end, with the running total carried.
__global__ __launch_bounds__(64) void gla_dg_kernel(const float* __restrict__ dG, float* __restrict__ dg, int T, int H) {
  const int lane = threadIdx.x, bh = blockIdx.x, b = bh / H, h = bh % H;
  const float* src = dG + (size_t)b * T * H + h;
  float* dst = dg + (size_t)b * T * H + h;
  float carry = 0.f;
  for (int t1 = T; t1 > 0; t1 -= 64) {
    const int t = t1 - 1 - lane;  // lane 0 takes the last token of the block
    float x = t >= 0 ? src[(size_t)t * H] : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (t >= 0) dst[(size_t)t * H] = x + carry;
    carry += __shfl(x, 63, 64);
  }
}

}  // namespace

hipError_t launch_gla_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                          const float* g, uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dg, void* workspace,
                          int B, int T, int H, float scale, hipStream_t stream) {
  const int N = (T + kC - 1) / kC;
  uint16_t* hs = (uint16_t*)workspace;
  uint16_t* dhs = hs + (size_t)B * H * N * kD * kD;
  float* dG = (float*)(dhs + (size_t)B * H * N * kD * kD);
  hipLaunchKernelGGL(gla_states_kernel, dim3(B * H, kD / 64, 2), dim3(256), 0, stream, q, k, v, dout, g, hs, dhs, T,
                     H, scale);
  hipLaunchKernelGGL(gla_dqkv_kernel, dim3(N, B * H), dim3(256), 0, stream, q, k, v, dout, g, hs, dhs, dq, dk, dv,
                     dG, T, H, scale);
  hipLaunchKernelGGL(gla_dg_kernel, dim3(B * H), dim3(64), 0, stream, dG, dg, T, H);
  return hipGetLastError();
}

size_t gla_bwd_workspace_bytes(int B, int T, int H) {
  const size_t N = (T + kC - 1) / kC;
  return 2 * (size_t)B * H * N * kD * kD * sizeof(uint16_t) + (size_t)B * T * H * sizeof(float);
}

}  // namespace mi355
