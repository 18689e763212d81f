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
// workgroup: dq, dk, dv and the per-token q.dq - k.dk, head-major in the
// workspace), gla_dg (reverse running sum over the sequence).
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
// A lane's element offsets are built once (Lofs); a 16-step of k or a
// 32-block of columns is an XOR of the offset and a block of rows an
// addition (the swizzle permutes 8-element slots by the row's low 4 bits).
template <int DT>
struct Lofs {
  int row, tr0, tr1;
  __device__ __forceinline__ explicit Lofs(int lane) {
    const int hi = lane >> 5, L = lane & 15, gp = (lane >> 4) & 1;
    row = swz_off<DT>(lane & 31, 4 * hi);
    const int col = 16 * gp + 4 * (L & 3);
    tr0 = swz_off<DT>(4 * hi + (L >> 2), col);
    tr1 = swz_off<DT>(8 + 4 * hi + (L >> 2), col);
  }
};
template <int DT>
__device__ __forceinline__ bf16x8 op_row(const uint16_t* t, const Lofs<DT>& o, int x0, int k0) {
  const int a = (o.row ^ k0) + x0 * DT;
  const u32x2 lo = *reinterpret_cast<const u32x2*>(t + a);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(t + (a ^ 8));
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}
template <int DT>
__device__ __forceinline__ bf16x8 op_tr(const uint16_t* t, const Lofs<DT>& o, int k0, int x0) {
  return lds_read_tr8(t + ((o.tr0 ^ x0) + k0 * DT), t + ((o.tr1 ^ x0) + k0 * DT));
}
// The k index (0..15 within a 16-step) of element i of a lane's operand.
__device__ __forceinline__ int op_k(int i, int hi) { return (i < 4 ? 4 * hi + i : 8 + 4 * hi + (i - 4)); }


// Inclusive running sum over the 64 lanes of one wave, into sG[0..63].
__device__ __forceinline__ void chunk_scan(float x, float* sG, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  sG[lane] = x;
}

// First chunk of a sweep: 0 forward, N-1 backward.
__device__ __forceinline__ int first_chunk(int dir, int N) { return dir ? N - 1 : 0; }

// Scale the 8 values of an operand by per-k factors f[k0 + op_k(i)].
__device__ __forceinline__ bf16x8 scale_op(bf16x8 v, const float* f, int k0, int hi) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; i++) x[i] = (float)v[i] * f[k0 + op_k(i, hi)];
  return pack8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
}

// ------------------------------------------------------------ chunk states
// Workgroup (b*H + h, dir): 8 waves own the 128 x 128 transposed state
// tile S^T (wave w: value rows 32(w & 3).., key columns 64(w >> 2) .., two
// 32x32 tiles; lane = key index, so each lane stores four consecutive values
// per 8-byte store).  Keeping the whole state in one workgroup reads each
// chunk's X once; the kernel moves about 1.1 GB per call on the benchmark
// workload and is bound by HBM bandwidth.
// dir 0 sweeps chunks forward and writes h_n (the state entering chunk n);
// dir 1 sweeps backward and writes dH_{n+1} (zero for the last chunk); both
// as [K][V] bf16.  Per chunk: X (k or q) and Y (v or do) arrive by LDS-DMA
// two chunks ahead; the update
// is S = exp(Gl) S + X^T (f o Y) with f_s = exp(Gl - G_s) (forward) or
// scale * exp(G_t) (backward), 0 past the end of the sequence.  The state
// stores stay in flight: each step waits only for its own tile loads.
__global__ __launch_bounds__(512) void gla_states_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const uint16_t* __restrict__ dout,
                                                         const float* __restrict__ g, uint16_t* __restrict__ hs,
                                                         uint16_t* __restrict__ dhs, int T, int H, float scale) {
  // Three buffers, chunk i of the sweep in buffer i % 3, loaded two steps
  // ahead.  A buffer's Y tile is followed by the chunk's raw g (64 fp32).
  // The loads are LDS-DMA issued as inline assembly and waited for
  // explicitly.
  constexpr int NW = 8;
  constexpr int kXT = kC * kD, kYT = kC * kD + 2 * kC;
  __shared__ __attribute__((aligned(16))) uint16_t sX[3 * kXT];
  __shared__ __attribute__((aligned(16))) uint16_t sY[3 * kYT];
  __shared__ float sG[NW][kC];  // per-wave copies: running sums of g, token factors
  __shared__ float sF[NW][kC];

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), hi = lane >> 5;
  const int bh = blockIdx.x, dir = blockIdx.z;
  const int b = bh / H, h = bh % H;
  const int N = (T + kC - 1) / kC;
  const size_t rs = (size_t)H * kD;
  const uint16_t* X = (dir ? q : k) + ((size_t)b * T * H + h) * kD;
  const uint16_t* Y = (dir ? dout : v) + ((size_t)b * T * H + h) * kD;
  const float* gb = g + (size_t)b * T * H + h;
  // N + 1 state slots per (b, h): slot N takes the state after the last
  // step, which nobody reads, so that every step stores (and loads)
  // unconditionally and the wait counts below hold on every path.
  uint16_t* out = (dir ? dhs : hs) + (size_t)bh * (N + 1) * kD * kD;
  const int vb = 32 * (w & 3), kb = 64 * (w >> 2);  // this wave's value rows, key columns
  const Lofs<kD> oD(lane);
  float* wG = sG[w];
  float* wF = sF[w];

  f32x16 acc[2] = {f32x16{}, f32x16{}};
  // Loads of a chunk: 2 + 2 instructions per wave, one more (g) for wave 0.
  auto load = [&](int n, int buf) {
    uint16_t* sx = sX + buf * kXT;
    uint16_t* sy = sY + buf * kYT;
    tile_load_async_asm<kD, kC, NW>(X, rs, n * kC, T, sx, w, lane);
    tile_load_async_asm<kD, kC, NW>(Y, rs, n * kC, T, sy, w, lane);
    if (w == 0) {  // g of the chunk (rows past the end repeat the last row; masked below)
      const int t = n * kC + min(lane, T - 1 - n * kC);
      dma_b32_asm(gb + (size_t)t * H, lds_addr(sy + kC * kD));
    }
  };
  // S^T element j of tile nb: value vb + c_row(j), key kb + 32nb + l32;
  // stored at [key][value], four consecutive values per store: one buffer
  // store instruction each, kStoreOps in all.
  constexpr int kStoreOps = 2 * 4;
  auto store = [&](int slot) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(out + (size_t)slot * kD * kD, (uint32_t)(kD * kD * 2));
    const uint32_t voff = (uint32_t)(((kb + (lane & 31)) * kD + vb + c_row(0, hi)) * 2);
#pragma unroll
    for (int nb = 0; nb < 2; nb++)
#pragma unroll
      for (int jg = 0; jg < 4; jg++) {
        const u32x2 v = u32x2{pack_bf16x2(acc[nb][4 * jg], acc[nb][4 * jg + 1]),
                              pack_bf16x2(acc[nb][4 * jg + 2], acc[nb][4 * jg + 3])};
        // c_row(4jg, hi) - c_row(0, hi) = 8jg values; tile nb is 32 keys further.
        __builtin_amdgcn_raw_buffer_store_b64(v, rs, voff, (int)((32 * nb * kD + 8 * jg) * 2), 0);
      }
  };
  // Order of a wave's vector-memory operations: loads of the first two
  // chunks (the initial state's store between them), then per step i the
  // loads of chunk i+2 (kLoadOps: the X and Y tiles; wave 0 adds one for
  // g, which only makes its waits below stricter) and the store of a state
  // (kStoreOps).  At step i >= 2, chunk i's loads are followed by a store,
  // chunk i+1's loads and another store; at steps 0 and 1 by a store and
  // one chunk's loads.  Waiting for "all but that many" is waiting for
  // chunk i.
  constexpr int kLoadOps = 2 * tile_load_ops<kD, kC, NW>();
  static_assert(kLoadOps == 4 && kStoreOps == 8, "wait counts below assume 4 loads and 8 stores per step");
  constexpr int kWaitLater = 2 * kStoreOps + kLoadOps, kWaitFirst = kStoreOps + kLoadOps;
  const int first = first_chunk(dir, N), stepn = dir ? -1 : 1;
  auto chunk_of = [&](int i) { return min(max(first + stepn * i, 0), N - 1); };  // past either end: a valid chunk
  load(chunk_of(0), 0);
  store(first);
  load(chunk_of(1), 1);
  for (int i = 0; i < N; i++) {
    const int n = first + stepn * i;
    const int buf = i % 3;
    const uint16_t* sx = sX + buf * kXT;
    const uint16_t* sy = sY + buf * kYT;
    const int nv = min(kC, T - n * kC);
    const int next = n + stepn;
    const int next_st = (next < 0 || next >= N) ? N : next;  // past either end: the spare slot
    if (i >= 2)
      wait_vmem_but<kWaitLater>();
    else
      wait_vmem_but<kWaitFirst>();
    lds_barrier();  // chunk n resident; every wave is done with step i-1 (and its buffer)
    // Every wave scans the chunk's g itself (no second barrier).
    chunk_scan(lane < nv ? reinterpret_cast<const float*>(sy + kC * kD)[lane] : 0.f, wG, lane);
    const float gl = wG[nv - 1];
    const float f = dir ? scale * __expf(wG[lane]) : __expf(gl - wG[lane]);
    wF[lane] = lane < nv ? f : 0.f;
    const float decay = __expf(gl);
    bf16x8 ao[kC / 16], bo[kC / 16][2];
#pragma unroll
    for (int ks = 0; ks < kC / 16; ks++) {
      ao[ks] = scale_op(op_tr<kD>(sy, oD, 16 * ks, vb), wF, 16 * ks, hi);
#pragma unroll
      for (int nb = 0; nb < 2; nb++) bo[ks][nb] = op_tr<kD>(sx, oD, 16 * ks, kb + 32 * nb);
    }
    asm volatile("" ::: "memory");
    load(chunk_of(i + 2), (i + 2) % 3);
#pragma unroll
    for (int nb = 0; nb < 2; nb++) acc[nb] *= decay;
#pragma unroll
    for (int ks = 0; ks < kC / 16; ks++)
#pragma unroll
      for (int nb = 0; nb < 2; nb++) acc[nb] = mfma32(ao[ks], bo[ks][nb], acc[nb]);
    store(next_st);
  }
  wait_vmem();  // the last loads (into buffers nobody reads) before the LDS goes away
}

// ------------------------------------------------------------ per-chunk stage
// Workgroup (chunk n, b*H + h), 8 waves.  LDS: q, k, v, do of the chunk
// [64][128], h_n and dH_{n+1} [128][128] (bf16, from the states kernel),
// the masked score matrices Mqk[t][s] = scale e^{G_t - G_s} (q_t.k_s) and
// Mdov[t][s] = scale e^{G_t - G_s} (do_t.v_s) for s <= t < nv (0 elsewhere).
// The outputs are computed transposed (dq^T [d][t], dk^T [d][s], dv^T
// [v][s]): a lane holds one token, so the state terms' per-token factors
// scale whole lanes, each lane writes four consecutive features per 8-byte
// store, and q.dq, k.dk are sums inside the lane.  Wave w owns feature rows
// 32(w >> 1) .. +31 and tokens 32(w & 1) .. +31 of each output.
// Outputs: dq, dk, dv (bf16) of the chunk's valid rows and
// dG_t = q_t.dq_t - k_t.dk_t (fp32), summed over the sequence by gla_dg.
__global__ __launch_bounds__(512) void gla_dqkv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ g, const uint16_t* __restrict__ hs,
                                                       const uint16_t* __restrict__ dhs, uint16_t* __restrict__ dq,
                                                       uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                                                       float* __restrict__ dG, int T, int H, float scale) {
  constexpr int NW = 8;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sK[kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sO[kC * kD];  // dO
  __shared__ __attribute__((aligned(16))) uint16_t sH[kD * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sDH[kD * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sMqk[kC * kC];
  __shared__ __attribute__((aligned(16))) uint16_t sMdov[kC * kC];
  __shared__ float sGr[kC];  // raw g of the chunk (LDS-DMA)
  __shared__ float sG[kC];
  __shared__ float sdG[2][4][kC];  // [q.dq or k.dk][feature block][token], each entry written once

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), hi = lane >> 5;
  const int l32 = lane & 31;
  const int n = blockIdx.x, bh = blockIdx.y;
  const int b = bh / H, h = bh % H;
  const int N = (T + kC - 1) / kC;
  const int nv = min(kC, T - n * kC);
  const size_t rs = (size_t)H * kD;
  const size_t base = ((size_t)b * T * H + h) * kD;
  const size_t st_off = ((size_t)bh * (N + 1) + n) * kD * kD;
  const Lofs<kD> oD(lane);
  const Lofs<kC> oC(lane);

  // Token tiles and g first, state tiles last, all by LDS-DMA issued as
  // inline assembly: the compiler adds no waits of its own, so the state
  // tiles keep arriving during the scan and the score products; the explicit
  // waits below (all but the 8 state-tile loads of this wave, then all) are
  // the only ones.
  tile_load_async_asm<kD, kC, NW>(q + base, rs, n * kC, T, sQ, w, lane);
  tile_load_async_asm<kD, kC, NW>(k + base, rs, n * kC, T, sK, w, lane);
  tile_load_async_asm<kD, kC, NW>(v + base, rs, n * kC, T, sV, w, lane);
  tile_load_async_asm<kD, kC, NW>(dout + base, rs, n * kC, T, sO, w, lane);
  if (w == 0) {  // rows past the end repeat the last row; masked in the scan
    const int t = n * kC + min(lane, nv - 1);
    dma_b32_asm(g + ((size_t)b * T + t) * H + h, lds_addr(sGr));
  }
  tile_load_async_asm<kD, kD, NW>(hs + st_off, kD, 0, kD, sH, w, lane);
  tile_load_async_asm<kD, kD, NW>(dhs + st_off, kD, 0, kD, sDH, w, lane);
  wait_vmem_but<8>();
  lds_barrier();
  if (w == 0) chunk_scan(lane < nv ? sGr[lane] : 0.f, sG, lane);
  lds_barrier();

  // Masked score matrices: wave w computes the 32x32 block (s-block
  // (w >> 1) & 1, t-block w & 1) of Mqk (w < 4) or Mdov (w >= 4), as
  // S^T[s][t] (A = k or v rows, B = q or do rows), and writes it
  // transposed, [t][s], four s values per 8-byte store.
  // (Each half of the waves names its tiles directly: a pointer chosen at
  // run time between LDS arrays hides from the compiler that these reads
  // cannot touch the state tiles still arriving.)
  auto scores = [&](const uint16_t* ta, const uint16_t* tb_, uint16_t* dst) {
    const int sb = (w >> 1) & 1, tb = w & 1;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kD / 16; ks++)
      acc = mfma32(op_row<kD>(ta, oD, 32 * sb, 16 * ks), op_row<kD>(tb_, oD, 32 * tb, 16 * ks), acc);
    const int t = 32 * tb + l32;
    const float gt = sG[t];
#pragma unroll
    for (int jg = 0; jg < 4; jg++) {
      float m[4];
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int s = 32 * sb + c_row(4 * jg + jj, hi);
        m[jj] = (s <= t && t < nv) ? acc[4 * jg + jj] * (scale * __expf(gt - sG[s])) : 0.f;
      }
      *reinterpret_cast<u32x2*>(dst + swz_off<kC>(t, 32 * sb + c_row(4 * jg, hi))) =
          u32x2{pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3])};
    }
  };
  if (w < 4)
    scores(sK, sQ, sMqk);
  else
    scores(sV, sO, sMdov);
  lds_barrier();

  const int fb = w >> 1, tb = w & 1;  // feature block (32 wide), token block
  const int tok = 32 * tb + l32;      // this lane's token
  const float gl = sG[nv - 1];

  // In-chunk products (transposed):
  //   dq^T[d][t] = sum_s k[s][d] Mdov[t][s]     dk^T[d][s] = sum_t q[t][d] Mdov[t][s]
  //   dv^T[v][s] = sum_t do[t][v] Mqk[t][s]
  f32x16 aq = f32x16{}, ak = f32x16{}, av = f32x16{};
#pragma unroll
  for (int ks = 0; ks < kC / 16; ks++) {
    aq = mfma32(op_tr<kD>(sK, oD, 16 * ks, 32 * fb), op_row<kC>(sMdov, oC, 32 * tb, 16 * ks), aq);
    ak = mfma32(op_tr<kD>(sQ, oD, 16 * ks, 32 * fb), op_tr<kC>(sMdov, oC, 16 * ks, 32 * tb), ak);
    av = mfma32(op_tr<kD>(sO, oD, 16 * ks, 32 * fb), op_tr<kC>(sMqk, oC, 16 * ks, 32 * tb), av);
  }
  wait_vmem();
  lds_barrier();  // h_n and dH_{n+1} resident
  // State terms (transposed), scaled per token (per lane):
  //   dq^T += scale e^{G_t} h do^T        dk^T += e^{Gl - G_s} dH v^T
  //   dv^T += e^{Gl - G_s} dH^T k^T
  f32x16 sq = f32x16{}, sk = f32x16{}, sv = f32x16{};
#pragma unroll
  for (int ks = 0; ks < kD / 16; ks++) {
    sq = mfma32(op_row<kD>(sH, oD, 32 * fb, 16 * ks), op_row<kD>(sO, oD, 32 * tb, 16 * ks), sq);
    sk = mfma32(op_row<kD>(sDH, oD, 32 * fb, 16 * ks), op_row<kD>(sV, oD, 32 * tb, 16 * ks), sk);
    sv = mfma32(op_tr<kD>(sDH, oD, 16 * ks, 32 * fb), op_row<kD>(sK, oD, 32 * tb, 16 * ks), sv);
  }
  const float fq = scale * __expf(sG[tok]), fkv = __expf(gl - sG[tok]);
  aq += fq * sq;
  ak += fkv * sk;
  av += fkv * sv;

  // q.dq and k.dk over this wave's 32 features: in-lane sums, the other
  // lane half, then one partial per (feature block, token) in LDS.
  float pq = 0.f, pk = 0.f;
#pragma unroll
  for (int jg = 0; jg < 4; jg++) {
    const int f0 = 32 * fb + c_row(4 * jg, hi);
    const u32x2 qv = *reinterpret_cast<const u32x2*>(sQ + swz_off<kD>(tok, f0));
    const u32x2 kv = *reinterpret_cast<const u32x2*>(sK + swz_off<kD>(tok, f0));
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const uint32_t wq = qv[jj >> 1], wk = kv[jj >> 1];
      const float xq = __uint_as_float((jj & 1) ? (wq & 0xffff0000u) : (wq << 16));
      const float xk = __uint_as_float((jj & 1) ? (wk & 0xffff0000u) : (wk << 16));
      pq = fmaf(xq, aq[4 * jg + jj], pq);
      pk = fmaf(xk, ak[4 * jg + jj], pk);
    }
  }
  pq = xhalf_sum(pq);
  pk = xhalf_sum(pk);
  if (hi == 0) {
    sdG[0][fb][tok] = pq;
    sdG[1][fb][tok] = pk;
  }
  lds_barrier();  // every wave is done with the state tiles; the q.dq / k.dk partials are complete
  // The outputs go out as whole rows: staged as bf16 [token][feature] tiles
  // (swizzled) in the state tiles' space, then copied with 16-byte stores,
  // each 256-byte row written by 16 consecutive lanes of one instruction.
  // (Rows assembled from 8-byte pieces of four waves reached HBM as partial
  // line writes, about 1.8 times the output bytes.)
  uint16_t* stq = sH;
  uint16_t* stk = sH + kC * kD;
  uint16_t* stv = sDH;
#pragma unroll
  for (int jg = 0; jg < 4; jg++) {
    const int o = swz_off<kD>(tok, 32 * fb + c_row(4 * jg, hi));
    *reinterpret_cast<u32x2*>(stq + o) = u32x2{pack_bf16x2(aq[4 * jg], aq[4 * jg + 1]),
                                               pack_bf16x2(aq[4 * jg + 2], aq[4 * jg + 3])};
    *reinterpret_cast<u32x2*>(stk + o) = u32x2{pack_bf16x2(ak[4 * jg], ak[4 * jg + 1]),
                                               pack_bf16x2(ak[4 * jg + 2], ak[4 * jg + 3])};
    *reinterpret_cast<u32x2*>(stv + o) = u32x2{pack_bf16x2(av[4 * jg], av[4 * jg + 1]),
                                               pack_bf16x2(av[4 * jg + 2], av[4 * jg + 3])};
  }
  if (w == 0 && lane < nv) {
    const float a = ((sdG[0][0][lane] + sdG[0][1][lane]) + (sdG[0][2][lane] + sdG[0][3][lane]));
    const float c = ((sdG[1][0][lane] + sdG[1][1][lane]) + (sdG[1][2][lane] + sdG[1][3][lane]));
    dG[(size_t)bh * T + n * kC + lane] = a - c;
  }
  lds_barrier();  // staged tiles complete
  {
    const int cs = lane & 15;
#pragma unroll
    for (int jj = 0; jj < 2; jj++) {
      const int r = 4 * (w + NW * jj) + (lane >> 4);  // token row of this lane
      if (r < nv) {
        const int o = swz_off<kD>(r, 8 * cs);
        const size_t g0 = base + (size_t)(n * kC + r) * rs + 8 * cs;
        *reinterpret_cast<u32x4*>(dq + g0) = *reinterpret_cast<const u32x4*>(stq + o);
        *reinterpret_cast<u32x4*>(dk + g0) = *reinterpret_cast<const u32x4*>(stk + o);
        *reinterpret_cast<u32x4*>(dv + g0) = *reinterpret_cast<const u32x4*>(stv + o);
      }
    }
  }
}

// dg[b, t, h] = sum_{t' >= t} dG[b*H + h][t']: one workgroup per (b, h),
// segments of 4096 tokens from the end (16 consecutive tokens per thread:
// in-thread suffix sums, then suffix sums of the thread totals across the
// wave (shuffles) and the four waves (LDS)), the running total carried.
__global__ __launch_bounds__(256) void gla_dg_kernel(const float* __restrict__ dG, float* __restrict__ dg, int T, int H) {
  constexpr int PER = 16, SEG = 256 * PER;
  __shared__ float sW[4];
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const float* src = dG + (size_t)bh * T;
  float* dst = dg + (size_t)b * T * H + h;
  float carry = 0.f;
  for (int seg_end = T; seg_end > 0; seg_end -= SEG) {
    const int t0 = seg_end - SEG + PER * tid;  // this thread's first token (may be negative)
    float x[PER];
    float tot = 0.f;
#pragma unroll
    for (int i = PER - 1; i >= 0; i--) {
      const int t = t0 + i;
      tot += (t >= 0 ? src[t] : 0.f);
      x[i] = tot;  // sum of this thread's tokens t0+i .. t0+PER-1
    }
    float suf = tot;  // inclusive suffix over the lanes of this wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_down(suf, o, 64);
      if (l + o < 64) suf += y;
    }
    if (l == 0) sW[w] = suf;
    __syncthreads();
    float after_w = 0.f;
    for (int j = w + 1; j < 4; j++) after_w += sW[j];
    const float seg_total = (sW[0] + sW[1]) + (sW[2] + sW[3]);
    const float after = suf - tot + after_w + carry;  // tokens after this thread's block
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const int t = t0 + i;
      if (t >= 0) dst[(size_t)t * H] = x[i] + after;
    }
    carry += seg_total;
    __syncthreads();  // sW reused by the next segment
  }
}

}  // namespace

hipError_t launch_gla_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                          const float* g, uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dg, void* workspace,
                          int B, int T, int H, float scale, hipStream_t stream) {
  const int N = (T + kC - 1) / kC;
  uint16_t* hs = (uint16_t*)workspace;
  uint16_t* dhs = hs + (size_t)B * H * (N + 1) * kD * kD;
  float* dG = (float*)(dhs + (size_t)B * H * (N + 1) * kD * kD);
  hipLaunchKernelGGL(gla_states_kernel, dim3(B * H, 1, 2), dim3(512), 0, stream, q, k, v, dout, g, hs, dhs, T, H,
                     scale);
  hipLaunchKernelGGL(gla_dqkv_kernel, dim3(N, B * H), dim3(512), 0, stream, q, k, v, dout, g, hs, dhs, dq, dk, dv,
                     dG, T, H, scale);
  hipLaunchKernelGGL(gla_dg_kernel, dim3(B * H), dim3(256), 0, stream, dG, dg, T, H);
  return hipGetLastError();
}

size_t gla_bwd_workspace_bytes(int B, int T, int H) {
  const size_t N = (T + kC - 1) / kC;
  return 2 * (size_t)B * H * (N + 1) * kD * kD * sizeof(uint16_t) + (size_t)B * T * H * sizeof(float);
}

}  // namespace mi355
