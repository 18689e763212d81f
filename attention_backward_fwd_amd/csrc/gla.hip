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
// (Gl: G at the chunk's last token).  Kernels: gla_sweep (per (b, h) one
// workgroup walks the chunks forward carrying h_n and writes dq, another
// walks them backward carrying dH_{n+1} and writes dk, dv; both keep the
// state on chip, so it never goes to HBM, and write the per-token q.dq and
// k.dk to the workspace), gla_dg (reverse running sum of
// q.dq - k.dk over the sequence).  This follows the page's account of where
// the gains come from: state kept on chip and HBM round trips cut.
#include "common.h"
#include "kernels.h"

namespace mi355 {

namespace {

constexpr int kC = 64;   // chunk length
constexpr int kD = 128;  // head dim (K = V)

// 32x32x16 operands from swizzled LDS tiles of DT-wide rows, in two k
// orders.  A product pairs operands of the same order:
//   op_row16 (tile stored [x][k], x = the lane's m or n index) and op_trc
//     (tile stored [k][x]): lane half hi gets k = 8hi .. 8hi+7;
//   op_tr (tile stored [k][x]): k = 4hi .. 4hi+3 and 8+4hi .. 8+4hi+3, the
//     order of the rows of a 32x32 result's elements 0..7, so it pairs with
//     operands taken straight from MFMA results.
// A lane's element offsets are built once (Lofs); a 16-step of k or a
// 32-block of columns is an XOR of the offset and a block of rows an
// addition (the swizzle permutes 8-element slots by the row's low 4 bits).
template <int DT>
struct Lofs {
  int row16, tr0, tr1, trc0, trc1;
  __device__ __forceinline__ explicit Lofs(int lane) {
    const int hi = lane >> 5, L = lane & 15, gp = (lane >> 4) & 1;
    row16 = swz_off<DT>(lane & 31, 8 * hi);
    const int col = 16 * gp + 4 * (L & 3);
    tr0 = swz_off<DT>(4 * hi + (L >> 2), col);
    tr1 = swz_off<DT>(8 + 4 * hi + (L >> 2), col);
    trc0 = swz_off<DT>(8 * hi + (L >> 2), col);
    trc1 = swz_off<DT>(8 * hi + 4 + (L >> 2), col);
  }
};
template <int DT>
__device__ __forceinline__ bf16x8 op_row16(const uint16_t* t, const Lofs<DT>& o, int x0, int k0) {
  return *reinterpret_cast<const bf16x8*>(t + ((o.row16 ^ k0) + x0 * DT));
}
template <int DT>
__device__ __forceinline__ bf16x8 op_tr(const uint16_t* t, const Lofs<DT>& o, int k0, int x0) {
  return lds_read_tr8(t + ((o.tr0 ^ x0) + k0 * DT), t + ((o.tr1 ^ x0) + k0 * DT));
}
template <int DT>
__device__ __forceinline__ bf16x8 op_trc(const uint16_t* t, const Lofs<DT>& o, int k0, int x0) {
  return lds_read_tr8(t + ((o.trc0 ^ x0) + k0 * DT), t + ((o.trc1 ^ x0) + k0 * DT));
}
// The k index (0..15 within a 16-step) of element i of a lane's operand.
__device__ __forceinline__ int op_k(int i, int hi) { return (i < 4 ? 4 * hi + i : 8 + 4 * hi + (i - 4)); }

// A chain of N products whose LDS operands are fetched PF - 1 steps ahead of
// the products that use them (fetch(k) returns step k's operands; use(k, ops)
// issues its products), one scheduling region per step.  Everything unrolls,
// so the operand array is registers.  One step ahead measured best here
// (deeper prefetch and split accumulation chains were no faster).
constexpr int kOpAhead = 2;  // PF of the chains below
template <int N, int PF, typename Fetch, typename Use>
__device__ __forceinline__ void pipelined(Fetch&& fetch, Use&& use) {
  decltype(fetch(0)) ops[N];
#pragma unroll
  for (int i = 0; i < PF - 1 && i < N; i++) ops[i] = fetch(i);
#pragma unroll
  for (int k = 0; k < N; k++) {
    if (k + PF - 1 < N) ops[k + PF - 1] = fetch(k + PF - 1);
    use(k, ops[k]);
    __builtin_amdgcn_sched_barrier(0);
  }
}
struct Ops2 {
  bf16x8 a, b;
};
struct Ops3 {
  bf16x8 a, b, c;
};
struct Ops4 {
  bf16x8 a, b, c, d;
};


// ------------------------------------------------------------ chunk sweeps
// One workgroup of 8 waves per (b*H + h, dir) walks the chunks of its
// sequence in order, dir 0 forward with h_n, dir 1 backward with dH_{n+1},
// and keeps that state on chip for the whole walk: fp32 in registers, as
// the transposed tile S^T[value][key] in the 32x32 MFMA result layout (wave
// w: value rows 32(w & 3).., key columns 64(w >> 2).., two tiles; lane = key
// index), and as a bf16 [key][value] copy in LDS that the state terms read.
// Per chunk, with its tiles arriving by LDS-DMA one chunk ahead (q, k, do
// double-buffered; v single-buffered, reloaded once every wave is past its
// last use):
//   dir 0: dq (in-chunk term from k and M_dov, state term from h_n and do),
//          q.dq per token, then h_{n+1};
//   dir 1: dk, dv (in-chunk terms from q, do and M_dov, M_qk; state terms
//          from dH_{n+1} and v, k), k.dk per token, then dH_n.
// The masked score tiles M_dov[t][s] = scale e^{G_t - G_s} (do_t . v_s) and
// M_qk[t][s] (s <= t) are formed once per chunk, one 32x32 tile per wave,
// in the result layout that is already the operand layout of the in-chunk
// products, and exchanged as ready-made operands (16 bytes per lane) through
// the state copy's LDS space, which the state terms have finished with by
// then.  Outputs are computed transposed (dq^T [d][t], dk^T [d][s], dv^T
// [v][s]; wave w: feature rows 32(w >> 1).., tokens 32(w & 1)..), so a lane
// holds one token and per-token factors scale whole lanes; they leave as
// whole rows through LDS staging.
//
// Every load is LDS-DMA and every store a buffer store, one instruction
// each, issued in a fixed order per step: the next chunk's q, k, do (and g,
// wave 0), its v after the first barrier, then this chunk's stores (kStF /
// kStB per wave, one more for wave 0); waiting for "all but the stores" at
// the top of a step is waiting for the chunk.  The chunk the last step
// loads is clamped to a valid one (never used).
constexpr int kStF = 2;      // dq (2 x 16 bytes of whole rows); wave 0 adds the q.dq store
constexpr int kStB = 2 * 2;  // dk, dv; wave 0 adds the k.dk store

// The value a wave-uniform lane holds (v_readlane: no LDS round trip).
__device__ __forceinline__ float lane_value(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Inclusive running sum over the 64 lanes of one wave, in DPP moves (no LDS
// round trips): running sums inside each row of 16 lanes (row_shr 1, 2, 4,
// 8; lanes shifted in from outside the row read 0), then the last lane of
// rows 0 and 2 added to rows 1 and 3 (row_bcast:15), then lane 31 to rows 2
// and 3 (row_bcast:31).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, true));
}
__device__ __forceinline__ float wave_scan(float x, int) {
  x += dpp_move<0x111, 0xf>(x);  // row_shr:1
  x += dpp_move<0x112, 0xf>(x);  // row_shr:2
  x += dpp_move<0x114, 0xf>(x);  // row_shr:4
  x += dpp_move<0x118, 0xf>(x);  // row_shr:8
  x += dpp_move<0x142, 0xa>(x);  // row_bcast:15 into rows 1, 3
  x += dpp_move<0x143, 0xc>(x);  // row_bcast:31 into rows 2, 3
  return x;
}

// Per-lane LDS offsets for one phase of a step: opaque copies of the base
// offsets behind a scheduling fence.  Every XOR-swizzled operand
// address is its own register; with the bases visible the compiler would
// compute all of them once, keep them across the chunk loop and spill.
__device__ __forceinline__ Lofs<kD> phase_lofs(const Lofs<kD>& b) {
  Lofs<kD> o = b;
  o.row16 = opaque_v(o.row16);
  o.tr0 = opaque_v(o.tr0);
  o.tr1 = opaque_v(o.tr1);
  o.trc0 = opaque_v(o.trc0);
  o.trc1 = opaque_v(o.trc1);
  __builtin_amdgcn_sched_barrier(0);
  return o;
}

template <int DIR>
__device__ __forceinline__ void gla_sweep(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                          const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                                          const float* __restrict__ g, uint16_t* __restrict__ dx0,
                                          uint16_t* __restrict__ dx1, float* __restrict__ dGp, int T, int H,
                                          float scale, uint16_t (*sQ)[kC * kD], uint16_t (*sK)[kC * kD],
                                          uint16_t* sV, uint16_t (*sO)[kC * kD], uint16_t* sS, float (*sG)[kC],
                                          float (*sD)[kC], float (*sW)[2][kC]) {
  constexpr int NW = 8;
  constexpr int kSt = DIR ? kStB : kStF;
  static_assert(tile_load_ops<kD, kC, NW>() == 2, "two LDS-DMA instructions per wave and tile");
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), hi = lane >> 5;
  const int l32 = lane & 31;
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int N = (T + kC - 1) / kC;
  const size_t rs = (size_t)H * kD;
  const size_t base = ((size_t)b * T * H + h) * kD;
  const int vb = 32 * (w & 3), kb = 64 * (w >> 2);  // state tiles of this wave
  const int fb = w >> 1, tb = w & 1;                // output tile: feature block, token block
  const int tok = 32 * tb + l32;                    // this lane's token within the chunk
  const Lofs<kD> lofs(lane);
  // Per-token values of this wave, read back by the lanes that need them
  // (16 bytes = 4 consecutive tokens per read): G of the chunk, and the
  // factors of the state update.
  float* wG = sW[w][0];
  float* wF = sW[w][1];
  // Score tiles, exchanged as ready-made MFMA operands through the state
  // copy's space while it is not in use: tile id, 32-token half, lane, 16
  // bytes each (2 KB per tile).
  bf16x8* sM = reinterpret_cast<bf16x8*>(sS);

  auto chunk_at = [&](int i) { return DIR ? N - 1 - min(i, N - 1) : min(i, N - 1); };
  // q, k, do of a chunk (double-buffered) and its g (wave 0; rows past the
  // end read the last row and are masked), issued after the step's scan;
  // v (single buffer) once every wave is done with it, after the step's
  // first barrier.  All are LDS-DMA, waited for explicitly.
  auto load_main = [&](int n, int buf) {
    tile_load_async_asm<kD, kC, NW>(q + base, rs, n * kC, T, sQ[buf], w, lane);
    tile_load_async_asm<kD, kC, NW>(k + base, rs, n * kC, T, sK[buf], w, lane);
    tile_load_async_asm<kD, kC, NW>(dout + base, rs, n * kC, T, sO[buf], w, lane);
    if (w == 0) dma_b32_asm(g + ((size_t)b * T + min(n * kC + lane, T - 1)) * H + h, lds_addr(sG[buf]));
  };
  auto load_v = [&](int n) { tile_load_async_asm<kD, kC, NW>(v + base, rs, n * kC, T, sV, w, lane); };

  // The state starts at zero: its bf16 copy too (made visible by the first
  // step's barrier).
  f32x16 st[2] = {f32x16{}, f32x16{}};
  auto store_state = [&]() {
#pragma unroll
    for (int nb = 0; nb < 2; nb++)
#pragma unroll
      for (int jg = 0; jg < 4; jg++) {
        const int key = kb + 32 * nb + l32;
        *reinterpret_cast<u32x2*>(sS + swz_off<kD>(key, vb + c_row(4 * jg, hi))) =
            u32x2{pack_bf16x2(st[nb][4 * jg], st[nb][4 * jg + 1]), pack_bf16x2(st[nb][4 * jg + 2], st[nb][4 * jg + 3])};
      }
  };
  store_state();
  load_main(chunk_at(0), 0);
  load_v(chunk_at(0));
  wait_vmem();

  for (int i = 0; i < N; i++) {
    const int n = chunk_at(i);
    const int buf = i & 1;
    const uint16_t* cQ = sQ[buf];
    const uint16_t* cK = sK[buf];
    const uint16_t* cV = sV;
    const uint16_t* cO = sO[buf];
    const int nv = min(kC, T - n * kC);
    // All but the previous step's stores: chunk n's tiles and g have landed.
    if (w == 0)
      wait_vmem_but<kSt + 1>();
    else
      wait_vmem_but<kSt>();
    lds_barrier();         // chunk n resident, the state copy complete; every wave is done with step i-1

    // G_t of the chunk in every lane t, its last value gl.
    const float Gl = wave_scan(lane < nv ? sG[buf][lane] : 0.f, lane);
    load_main(chunk_at(i + 1), buf ^ 1);
    wG[lane] = Gl;
    const float gl = lane_value(Gl, nv - 1);
    const float decay = __expf(gl);
    const float G_tok = wG[tok];

    // 32x32 product over the 128 features of rows 32 ra.. of ta and rows
    // 32 rb.. of tb_: row = ta's token, column (lane) = tb_'s token.
    auto score = [&](const uint16_t* ta, int ra, const uint16_t* tb_, int rb) {
      const Lofs<kD> oD = phase_lofs(lofs);
      f32x16 acc = f32x16{};
      pipelined<kD / 16, kOpAhead>(
          [&](int ks) { return Ops2{op_row16<kD>(ta, oD, 32 * ra, 16 * ks), op_row16<kD>(tb_, oD, 32 * rb, 16 * ks)}; },
          [&](int, const Ops2& o) { acc = mfma32(o.a, o.b, acc); });
      return acc;
    };
    // Mask and scale of a score tile whose lanes are the tokens 32 lb.. and
    // registers the tokens 32 rb + c_row(j): scale e^{G_t - G_s} for s <= t
    // (dir 0: lane = t, register = s; dir 1: lane = s, register = t), t
    // within the chunk, else 0; then the tile's two 16-token operand halves
    // go to the exchange area as tile `id`.
    auto publish = [&](const f32x16& acc, int lb, int rb, int id) {
      const int own = 32 * lb + l32;
      const float G_own = wG[own];
      float f[16];
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int oth = 32 * rb + c_row(j, hi);
        const float G_oth = reinterpret_cast<const f32x4*>(wG + 32 * rb + c_row(4 * (j >> 2), hi))[0][j & 3];
        const bool keep = DIR ? (own <= oth && oth < nv) : (oth <= own && own < nv);
        f[j] = keep ? scale * __expf(DIR ? G_oth - G_own : G_own - G_oth) : 0.f;
      }
#pragma unroll
      for (int hh = 0; hh < 2; hh++) {
        const int o = 8 * hh;
        sM[(2 * id + hh) * 64 + lane] =
            pack8(acc[o] * f[o], acc[o + 1] * f[o + 1], acc[o + 2] * f[o + 2], acc[o + 3] * f[o + 3],
                  acc[o + 4] * f[o + 4], acc[o + 5] * f[o + 5], acc[o + 6] * f[o + 6], acc[o + 7] * f[o + 7]);
      }
    };
    // Per-token factor of a state update for the 8 tokens of operand k-step
    // ks (from wF: tokens 16 ks + op_k(e), two runs of four).
    auto scale_by = [&](bf16x8 x, int ks) {
      const f32x4 f0 = *reinterpret_cast<const f32x4*>(wF + 16 * ks + op_k(0, hi));
      const f32x4 f1 = *reinterpret_cast<const f32x4*>(wF + 16 * ks + op_k(4, hi));
      return pack8((float)x[0] * f0[0], (float)x[1] * f0[1], (float)x[2] * f0[2], (float)x[3] * f0[3],
                   (float)x[4] * f1[0], (float)x[5] * f1[1], (float)x[6] * f1[2], (float)x[7] * f1[3]);
    };
    // State update: st^T[value][key] = e^{gl} st^T + sum_x f_x ty[x][value] tx[x][key].
    auto update = [&](const uint16_t* ty, const uint16_t* tx, float f_lane) {
      wF[lane] = f_lane;
      const Lofs<kD> oD = phase_lofs(lofs);
#pragma unroll
      for (int nb = 0; nb < 2; nb++) st[nb] *= decay;
      pipelined<kC / 16, kOpAhead>(
          [&](int ks) {
            return Ops3{op_tr<kD>(ty, oD, 16 * ks, vb), op_tr<kD>(tx, oD, 16 * ks, kb), op_tr<kD>(tx, oD, 16 * ks, kb + 32)};
          },
          [&](int ks, const Ops3& o) {
            const bf16x8 a = scale_by(o.a, ks);
            st[0] = mfma32(a, o.b, st[0]);
            st[1] = mfma32(a, o.c, st[1]);
          });
    };

    // Outputs leave as whole rows: a wave puts its 32 tokens x 32 features
    // into a staging tile ([token][feature], swizzled like the input tiles;
    // four features per 8-byte write), and after a barrier each wave copies
    // 8 of the 64 rows out, 16 lanes per 256-byte row (two 16-byte stores
    // per lane).  Rows past the end of the sequence fall outside the buffer
    // range and are dropped.
    auto stage = [&](uint16_t* tile, const f32x16& a) {
#pragma unroll
      for (int jg = 0; jg < 4; jg++)
        *reinterpret_cast<u32x2*>(tile + swz_off<kD>(tok, 32 * fb + c_row(4 * jg, hi))) =
            u32x2{pack_bf16x2(a[4 * jg], a[4 * jg + 1]), pack_bf16x2(a[4 * jg + 2], a[4 * jg + 3])};
    };
    auto store_rows = [&](uint16_t* dst, const uint16_t* tile) {
      const __amdgpu_buffer_rsrc_t ro =
          buffer_rsrc(dst + base + (size_t)n * kC * rs, (uint32_t)(((size_t)(nv - 1) * rs + kD) * 2));
      const int cs = lane & 15;
#pragma unroll
      for (int jj = 0; jj < 2; jj++) {
        const int r = 4 * (w + NW * jj) + (lane >> 4);  // token row of this lane
        const u32x4 x = *reinterpret_cast<const u32x4*>(tile + swz_off<kD>(r, 8 * cs));
        __builtin_amdgcn_raw_buffer_store_b128(x, ro, (uint32_t)(((size_t)r * rs + 8 * cs) * 2), 0, 0);
      }
    };
    // x_t . d_t over this wave's 32 features (x from the chunk tile) into
    // LDS, one partial per (feature block, token); after the next barrier
    // wave 0 sums the four in a fixed order and writes dGp[DIR][bh][t].
    auto dot_partial = [&](const uint16_t* tx, const f32x16& a) {
      float p = 0.f;
#pragma unroll
      for (int jg = 0; jg < 4; jg++) {
        const u32x2 xv = *reinterpret_cast<const u32x2*>(tx + swz_off<kD>(tok, 32 * fb + c_row(4 * jg, hi)));
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const uint32_t wx = xv[jj >> 1];
          p = fmaf(__uint_as_float((jj & 1) ? (wx & 0xffff0000u) : (wx << 16)), a[4 * jg + jj], p);
        }
      }
      p = xhalf_sum(p);
      if (hi == 0) sD[fb][tok] = p;
    };
    auto store_dot = [&]() {
      if (w == 0) {
        const float x = (sD[0][lane] + sD[1][lane]) + (sD[2][lane] + sD[3][lane]);
        const __amdgpu_buffer_rsrc_t rd =
            buffer_rsrc(dGp + ((size_t)DIR * gridDim.x + bh) * T + (size_t)n * kC, (uint32_t)(nv * 4));
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rd, (uint32_t)(lane * 4), 0, 0);
      }
    };

    // Phases of a step: (S) state terms, reading the state copy; (M) score
    // tiles, one per wave (dir 0: four tiles; there every wave also updates
    // the state here); barrier; the next chunk's v goes out, the tiles
    // replace the state copy; barrier; (I) in-chunk terms, outputs staged
    // (dir 1: then the state update); barrier; rows out (dir 1: barrier);
    // the new state copy.
    if constexpr (DIR == 0) {
      // dq^T[d][t] = scale e^{G_t} sum_v h[d][v] do[t][v] + sum_s k[s][d] M_dov[t][s]
      f32x16 aq = f32x16{};
      {
        const Lofs<kD> oD = phase_lofs(lofs);
        pipelined<kD / 16, kOpAhead>(
            [&](int ks) { return Ops2{op_row16<kD>(sS, oD, 32 * fb, 16 * ks), op_row16<kD>(cO, oD, 32 * tb, 16 * ks)}; },
            [&](int, const Ops2& o) { aq = mfma32(o.a, o.b, aq); });
      }
      aq *= scale * __expf(G_tok);
      // h_{n+1} = e^{gl} h_n + sum_s e^{gl - G_s} k_s^T v_s (s < nv)
      const float f_lane = lane < nv ? __expf(gl - Gl) : 0.f;
      f32x16 m;
      if (w < 4) m = score(cV, w >> 1, cO, w & 1);  // M_dov^T[s][t]: s block w >> 1, t block w & 1
      update(cV, cK, f_lane);
      lds_barrier();  // every wave is done with the state copy and with v
      load_v(chunk_at(i + 1));
      if (w < 4) publish(m, w & 1, w >> 1, w);
      lds_barrier();  // score tiles complete
      {
        const Lofs<kD> oD = phase_lofs(lofs);
        pipelined<kC / 16, kOpAhead>(
            [&](int ks) {
              return Ops2{op_tr<kD>(cK, oD, 16 * ks, 32 * fb), sM[(2 * ((ks >> 1) * 2 + tb) + (ks & 1)) * 64 + lane]};
            },
            [&](int, const Ops2& o) { aq = mfma32(o.a, o.b, aq); });
      }
      dot_partial(cQ, aq);
      // dq is staged where this wave's lanes just read q (no other wave reads
      // the q tile after the first barrier).
      uint16_t* tq = sQ[buf];
      stage(tq, aq);
      lds_barrier();  // staged rows and dot partials complete; every wave is done with the score tiles
      store_rows(dx0, tq);
      store_dot();
    } else {
      // dk^T[d][s] = e^{gl - G_s} sum_v dH[d][v] v[s][v] + sum_t q[t][d] M_dov[t][s]
      // dv^T[v][s] = e^{gl - G_s} sum_k dH[k][v] k[s][k] + sum_t do[t][v] M_qk[t][s]
      f32x16 ak = f32x16{}, av = f32x16{};
      {
        const Lofs<kD> oD = phase_lofs(lofs);
        pipelined<kD / 16, kOpAhead>(
            [&](int ks) {
              return Ops4{op_row16<kD>(sS, oD, 32 * fb, 16 * ks), op_row16<kD>(cV, oD, 32 * tb, 16 * ks),
                          op_trc<kD>(sS, oD, 16 * ks, 32 * fb), op_row16<kD>(cK, oD, 32 * tb, 16 * ks)};
            },
            [&](int, const Ops4& o) {
              ak = mfma32(o.a, o.b, ak);
              av = mfma32(o.c, o.d, av);
            });
      }
      const float fkv = __expf(gl - G_tok);
      ak *= fkv;
      av *= fkv;
      // Tile w: type w >> 2 (M_dov, M_qk), t block (w >> 1) & 1, s block w & 1.
      const f32x16 m = (w >> 2) ? score(cQ, (w >> 1) & 1, cK, w & 1) : score(cO, (w >> 1) & 1, cV, w & 1);
      lds_barrier();  // every wave is done with the state copy and with v
      load_v(chunk_at(i + 1));
      publish(m, w & 1, (w >> 1) & 1, w);
      lds_barrier();  // score tiles complete
      {
        const Lofs<kD> oD = phase_lofs(lofs);
        pipelined<kC / 16, kOpAhead>(
            [&](int ks) {
              const int id = (ks >> 1) * 2 + tb;
              return Ops4{op_tr<kD>(cQ, oD, 16 * ks, 32 * fb), sM[(2 * id + (ks & 1)) * 64 + lane],
                          op_tr<kD>(cO, oD, 16 * ks, 32 * fb), sM[(2 * (4 + id) + (ks & 1)) * 64 + lane]};
            },
            [&](int, const Ops4& o) {
              ak = mfma32(o.a, o.b, ak);
              av = mfma32(o.c, o.d, av);
            });
      }
      dot_partial(cK, ak);
      // dk is staged where this wave's lanes just read k (no other wave reads
      // the k tile after the first barrier), dv in the half of the state
      // copy's space the score tiles leave free.
      uint16_t* tk = sK[buf];
      uint16_t* tv = sS + kC * kD;
      stage(tk, ak);
      stage(tv, av);
      // dH_n = e^{gl} dH_{n+1} + scale sum_t e^{G_t} q_t^T do_t (t < nv)
      update(cO, cQ, lane < nv ? scale * __expf(Gl) : 0.f);
      lds_barrier();  // staged rows and dot partials complete; every wave is done with the score tiles
      store_rows(dx0, tk);
      store_rows(dx1, tv);
      store_dot();
      lds_barrier();  // every wave is done with the staged dv
    }
    store_state();
  }
  wait_vmem();  // the last loads (into buffers nobody reads) before the LDS goes away
}

__global__ __launch_bounds__(512) void gla_sweep_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v,
                                                        const uint16_t* __restrict__ dout,
                                                        const float* __restrict__ g, uint16_t* __restrict__ dq,
                                                        uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                                                        float* __restrict__ dGp, int T, int H, float scale) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sO[2][kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kC * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sS[kD * kD];
  __shared__ __attribute__((aligned(16))) float sG[2][kC];
  __shared__ __attribute__((aligned(16))) float sD[4][kC];
  __shared__ __attribute__((aligned(16))) float sW[8][2][kC];
  if (blockIdx.y == 0)
    gla_sweep<0>(q, k, v, dout, g, dq, nullptr, dGp, T, H, scale, sQ, sK, sV, sO, sS, sG, sD, sW);
  else
    gla_sweep<1>(q, k, v, dout, g, dk, dv, dGp, T, H, scale, sQ, sK, sV, sO, sS, sG, sD, sW);
}

// dg[b, t, h] = sum_{t' >= t} dG_{t'} with dG_t = q_t.dq_t - k_t.dk_t.  One
// workgroup per (b, 4 consecutive heads, segment of 1024 tokens counted from
// the end), 256 threads per head, 4 consecutive tokens per thread: the sum
// of all tokens after the segment (each thread a fixed strided share, then
// a fixed reduction tree), in-thread suffix sums, and an exclusive suffix
// over the 256 thread totals of a head (one wave per head, four totals per
// lane, shuffles).  The threads of a head group are interleaved so that each
// store covers 4 heads of a token (16 contiguous bytes of dg).
constexpr int kDgHeads = 4, kDgThreads = 256, kDgPer = 4, kDgSeg = kDgThreads * kDgPer;
__global__ __launch_bounds__(kDgHeads * kDgThreads) void gla_dg_kernel(const float* __restrict__ dGp,
                                                                        float* __restrict__ dg, int T, int H,
                                                                        int BH) {
  constexpr int NPL = kDgThreads / 64;                 // totals per lane in the head scan
  constexpr int NWV = kDgHeads * kDgThreads / 64;     // waves of the workgroup
  __shared__ float sT[kDgHeads][kDgThreads];
  __shared__ float sTot[kDgHeads][NWV];
  const int tid = threadIdx.x, hl = tid % kDgHeads, tq = tid / kDgHeads;
  const int lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x, h = blockIdx.y * kDgHeads + hl;
  const bool on = h < H;
  const int bh = b * H + (on ? h : 0);
  const float* pq = dGp + (size_t)bh * T;
  const float* pk = dGp + ((size_t)BH + bh) * T;
  float* dst = dg + (size_t)b * T * H + h;
  const int seg_end = T - (int)blockIdx.z * kDgSeg;
  const bool vec = (T & 3) == 0;
  auto load4 = [&](int t0, float (&x)[kDgPer]) {
    if (vec && t0 >= 0 && t0 + 4 <= T) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(pq + t0);
      const f32x4 c = *reinterpret_cast<const f32x4*>(pk + t0);
#pragma unroll
      for (int i = 0; i < 4; i++) x[i] = a[i] - c[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int t = t0 + i;
        x[i] = (t >= 0 && t < T) ? pq[t] - pk[t] : 0.f;
      }
    }
  };
  // Tokens after the segment: this thread's share, then the head's sum.
  float after_seg = 0.f;
  for (int t0 = seg_end + kDgPer * tq; t0 < T; t0 += kDgSeg) {
    float y[kDgPer];
    load4(t0, y);
    after_seg += (y[0] + y[1]) + (y[2] + y[3]);
  }
#pragma unroll
  for (int o = kDgHeads; o < 64; o <<= 1) after_seg += __shfl_xor(after_seg, o, 64);
  if (lane < kDgHeads) sTot[lane][w] = after_seg;  // lane == hl here; w < NWV
  // This segment.
  const int t0 = seg_end - kDgSeg + kDgPer * tq;  // this thread's first token (may be negative)
  float x[kDgPer];
  load4(t0, x);
  float tot = 0.f;
#pragma unroll
  for (int i = kDgPer - 1; i >= 0; i--) {
    tot += x[i];
    x[i] = tot;  // sum of this thread's tokens t0+i .. t0+kDgPer-1
  }
  sT[hl][tq] = tot;
  __syncthreads();
  float carry = 0.f;
#pragma unroll
  for (int i = 0; i < NWV; i++) carry += sTot[hl][i];
  if (w < kDgHeads) {  // wave w: exclusive suffix over the totals of head w
    float a[NPL], part = 0.f;
#pragma unroll
    for (int i = NPL - 1; i >= 0; i--) {
      a[i] = sT[w][NPL * lane + i];
      part += a[i];
    }
    float suf = part;  // inclusive suffix over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_down(suf, o, 64);
      if (lane + o < 64) suf += y;
    }
    float run = suf - part;
#pragma unroll
    for (int i = NPL - 1; i >= 0; i--) {
      sT[w][NPL * lane + i] = run;
      run += a[i];
    }
  }
  __syncthreads();
  const float after = sT[hl][tq] + carry;  // tokens of this head after this thread's block
  if (on) {
#pragma unroll
    for (int i = 0; i < kDgPer; i++) {
      const int t = t0 + i;
      if (t >= 0) dst[(size_t)t * H] = x[i] + after;
    }
  }
}

}  // namespace

hipError_t launch_gla_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                          const float* g, uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dg, void* workspace,
                          int B, int T, int H, float scale, hipStream_t stream) {
  float* dGp = (float*)workspace;
  hipLaunchKernelGGL(gla_sweep_kernel, dim3(B * H, 2), dim3(512), 0, stream, q, k, v, dout, g, dq, dk, dv, dGp, T,
                     H, scale);
  hipLaunchKernelGGL(gla_dg_kernel, dim3(B, (H + kDgHeads - 1) / kDgHeads, (T + kDgSeg - 1) / kDgSeg),
                     dim3(kDgHeads * kDgThreads), 0, stream, dGp, dg, T, H, B * H);
  return hipGetLastError();
}

size_t gla_bwd_workspace_bytes(int B, int T, int H) { return 2 * (size_t)B * H * T * sizeof(float); }

}  // namespace mi355
