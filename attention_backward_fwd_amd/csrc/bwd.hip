// Backward of exact softmax attention on gfx950 (dQ, dK, dV).
//
// Decomposition as in the FlashAttention backward examples of TileLang #940
// (flashattn_bwd_atomic_add / flashattn_bwd_split): one workgroup owns a block
// of 128 keys of one (batch, query head), keeps its dK/dV accumulators on
// chip for the whole sweep and walks the query blocks that see those keys.
// Per 64-query block the five tile contractions run on the matrix cores:
//
//   S  = Q K^T            A = Q (LDS, row reads)      B = K (LDS, row reads)
//   dP = dO V^T           A = dO (LDS, row reads)     B = V (LDS, row reads)
//   dV += P^T dO          A = P^T (registers)         B = dO (LDS, transposing reads)
//   dK += dS^T Q          A = dS^T (registers)        B = Q (LDS, transposing reads)
//   dQ  = dS K            A = dS (LDS, transposing)   B = K (LDS, transposing reads)
//
// with P recomputed from the forward's LSE and dS = P o (dP - Delta).  The
// 32x32 MFMA result layout puts one key in each lane and 16 query rows in its
// registers; that is already the A-operand layout of P^T and dS^T for the dV
// and dK products, so those never leave registers.  dQ needs dS with queries
// in lanes, so dS^T goes through LDS.
//
// The softmax scale is folded into the exponent: the kernel forms
// P' = scale * P = exp2(S*scale*log2e - (LSE*log2e - log2(scale))), so that
// dS' = P' o (dP - Delta) = scale * dS is what both dQ and dK need; only dV
// is divided by the scale, once, at the end.
//
// Q and dO blocks are double-buffered in LDS and filled by LDS-DMA loads
// issued one block ahead; two workgroup barriers per query block.
//
// dQ leaves the workgroup either as fp32 atomic adds into one accumulator
// (the page's atomic variant, with fp32 rather than bf16 atomics) or as a
// plain store into this key block's own fp32 partial slot, summed later in a
// fixed order by dq_sum_kernel (the split+sum variant): every partial element
// has exactly one writer, which makes that path bitwise deterministic.
//
// dK/dV never use atomics.  With one query head per KV head they are written
// as bf16 here; with grouped-query attention each query head writes an fp32
// partial and the postprocess sums a group's partials in a fixed order.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mi355 {

namespace {

constexpr int kBN = kBwdBlockN;  // keys per workgroup (4 waves x 32)
constexpr int kBM = 64;          // queries per step

template <int D, bool CAUSAL, bool ATOMIC, bool PARTIAL>
__global__ __launch_bounds__(256) void bwd_kernel(BwdParams p) {
  constexpr int BN = kBN, BM = kBM;
  constexpr int TQ = BM * D;  // elements of one Q or dO block
  constexpr int NKS = D / 16, NDT = D / 32;
  // dQ tile split over the 4 waves: D=128 -> one 32-wide d tile and both
  // 32-row query tiles per wave; D=64 -> one 32x32 tile per wave.
  constexpr int DQ_MT = (D == 128) ? 2 : 1;

  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2 * TQ];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[2 * TQ];
  __shared__ __attribute__((aligned(16))) uint16_t sdSt[BN * BM];  // dS'^T [key][query], swizzled
  __shared__ __attribute__((aligned(16))) float sL[2 * BM];
  __shared__ __attribute__((aligned(16))) float sDl[2 * BM];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hi = lane >> 5, l32 = lane & 31, L = lane & 15, Gp = (lane >> 4) & 1;
  const int S = p.S, Hq = p.Hq, G = p.G, Hkv = p.Hkv;
  const int n_nblk = (S + BN - 1) / BN;

  // Tile order: each XCD gets a contiguous range of (batch, KV head) groups
  // and works through them one at a time (their Q/dO rows stay in its L2);
  // inside a group, key blocks run heaviest-first (block 0 sees every query
  // under causal masking) with the group's query heads side by side.
  const int nwg = gridDim.x, NG = p.B * Hkv;
  int t = blockIdx.x, x = 0, NGx = NG;
  if (NG % 8 == 0) {
    t = xcd_remap(blockIdx.x, nwg);
    const int per = nwg / 8;
    x = t / per;
    t -= x * per;
    NGx = NG / 8;
  }
  const int per_group = n_nblk * G;
  const int grp = x * NGx + t / per_group;
  const int jb = (t % per_group) / G;
  const int r = t % G;
  const int b = grp / Hkv, kvh = grp % Hkv, h = kvh * G + r;
  const int n0 = jb * BN;

  const size_t qrs = (size_t)Hq * D, kvrs = (size_t)Hkv * D;
  const uint16_t* Qb = p.q + ((size_t)b * S * Hq + h) * D;
  const uint16_t* dOb = p.dout + ((size_t)b * S * Hq + h) * D;
  const uint16_t* Kb = p.k + ((size_t)b * S * Hkv + kvh) * D;
  const uint16_t* Vb = p.v + ((size_t)b * S * Hkv + kvh) * D;
  const float* lse_b = p.lse + (size_t)(b * Hq + h) * S;
  const float* dl_b = p.delta + (size_t)(b * Hq + h) * S;

  const float c = p.scale * kLog2e;
  const float lsc = __builtin_amdgcn_logf(p.scale);  // log2(scale)
  const int m_begin = CAUSAL ? n0 : 0;               // n0 is a multiple of BM
  const int n_steps = (S - m_begin + BM - 1) / BM;

  float lr = 0.f, dlr = 0.f;
  auto load_rows = [&](int m0) {
    if (tid < BM) {
      const int q = m0 + tid;
      // Rows past the end get +inf, so P = 0 there without a mask.
      lr = q < S ? fmaf(lse_b[q], kLog2e, -lsc) : INFINITY;
      dlr = q < S ? dl_b[q] : 0.f;
    }
  };
  // Key/value block (resident for the whole sweep) and the first Q/dO block.
  tile_load_async<D, BN>(Kb, kvrs, n0, S, sK, w, lane);
  tile_load_async<D, BN>(Vb, kvrs, n0, S, sV, w, lane);
  tile_load_async<D, BM>(Qb, qrs, m_begin, S, sQ, w, lane);
  tile_load_async<D, BM>(dOb, qrs, m_begin, S, sdO, w, lane);
  load_rows(m_begin);

  // Per-lane LDS element offsets; the loops derive the rest with XORs of
  // column moves and additions of 16-row moves (see xslot()).
  const int offR0 = swz_off<D>(l32, 8 * hi);         // 16-byte row reads, row l32
  const int offKV0 = offR0 + 32 * w * D;              //   ... row 32w + l32 (this wave's keys)
  const int tcol = 16 * Gp + 4 * (L & 3);
  const int offT00 = swz_off<D>(4 * hi + (L >> 2), tcol);      // transposing reads of Q / dO
  const int offT10 = swz_off<D>(4 * hi + (L >> 2) + 8, tcol);
  const int dq_nt = (D == 128) ? w : (w & 1);
  const int dq_mt0 = (D == 128) ? 0 : (w >> 1);
  const int offK00 = swz_off<D>(8 * hi + (L >> 2), 32 * dq_nt + tcol);  // transposing reads of K
  const int offK10 = swz_off<D>(8 * hi + (L >> 2) + 4, 32 * dq_nt + tcol);
  const int offS00 = swz_off<BM>(8 * hi + (L >> 2), tcol);     // transposing reads of dS'^T
  const int offS10 = swz_off<BM>(8 * hi + (L >> 2) + 4, tcol);
  const int offW0 = swz_off<BM>(32 * w + l32, 4 * hi);         // 8-byte writes of dS'^T

  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; dt++) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }
  const int key_l = n0 + 32 * w + l32;
  const int dq_d = 32 * dq_nt + l32;
  const uint32_t row_bytes = (uint32_t)(Hq * D) * 4u;
  const uint32_t dq_voff = (uint32_t)(4 * hi) * row_bytes + (uint32_t)dq_d * 4u;
  const size_t nq = (size_t)p.B * S * Hq * D;

  for (int st = 0; st < n_steps; st++) {
    const int buf = st & 1;
    const int m0 = m_begin + st * BM;
    if (tid < BM) {
      sL[buf * BM + tid] = lr;
      sDl[buf * BM + tid] = dlr;
    }
    wait_vmem();
    __syncthreads();  // block st resident; every wave is done with step st-1
    if (st + 1 < n_steps) {
      tile_load_async<D, BM>(Qb, qrs, m0 + BM, S, sQ + (buf ^ 1) * TQ, w, lane);
      tile_load_async<D, BM>(dOb, qrs, m0 + BM, S, sdO + (buf ^ 1) * TQ, w, lane);
      load_rows(m0 + BM);
    }
    const uint16_t* cQ = sQ + buf * TQ;
    const uint16_t* cdO = sdO + buf * TQ;
    const float* cL = sL + buf * BM;
    const float* cDl = sDl + buf * BM;
    // Recompute the LDS addresses every step (one XOR each) rather than
    // keeping dozens of them live across the loop.
    const int offR = opaque_v(offR0), offKV = opaque_v(offKV0), offT0 = opaque_v(offT00),
              offT1 = opaque_v(offT10), offK0 = opaque_v(offK00), offK1 = opaque_v(offK10),
              offS0 = opaque_v(offS00), offS1 = opaque_v(offS10), offW = opaque_v(offW0);

    // Two 32-query halves in turn: S, dP, softmax, dS'^T to LDS and the
    // dV/dK updates of the first half are independent of the second half's
    // products, so the scheduler can overlap them.
    const bool need_mask = (n0 + BN > S) || (CAUSAL && m0 < n0 + BN);
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys.
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ks++) {
        const int o = xslot(offR, 16 * ks) + 32 * mt * D;
        s = mfma32(lds_read_b128(cQ + o), lds_read_b128(sK + xslot(offKV, 16 * ks)), s);
        dp = mfma32(lds_read_b128(cdO + o), lds_read_b128(sV + xslot(offKV, 16 * ks)), dp);
      }
      // P' = scale P and dS' = scale dS.  Element j of lane l is query
      // 32mt + 8(j/4) + 4hi + j%4 of the block, key 32w + l32.
      uint32_t pp[8], dd[8];
#pragma unroll
      for (int jg = 0; jg < 4; jg++) {
        const int qo = 32 * mt + 8 * jg + 4 * hi;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(cL + qo);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(cDl + qo);
        float pv[4], dv4[4];
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int j = 4 * jg + jj;
          float e = __builtin_amdgcn_exp2f(fmaf(s[j], c, -l4[jj]));
          const int q = m0 + qo + jj;
          e = (need_mask && (key_l >= S || (CAUSAL && key_l > q))) ? 0.f : e;
          pv[jj] = e;
          dv4[jj] = e * (dp[j] - d4[jj]);
        }
        pp[2 * jg] = pack_bf16x2(pv[0], pv[1]);
        pp[2 * jg + 1] = pack_bf16x2(pv[2], pv[3]);
        dd[2 * jg] = pack_bf16x2(dv4[0], dv4[1]);
        dd[2 * jg + 1] = pack_bf16x2(dv4[2], dv4[3]);
      }
      // dS'^T to LDS as [key][query] (a 64-wide swizzled tile): four
      // consecutive queries per 8-byte write.
#pragma unroll
      for (int jg = 0; jg < 4; jg++)
        *reinterpret_cast<u32x2*>(sdSt + xslot(offW, 8 * jg + 32 * mt)) = u32x2{dd[2 * jg], dd[2 * jg + 1]};
      // dV += P'^T dO and dK += dS'^T Q; the B operands are columns of dO
      // and Q, fetched with transposing LDS reads in the query order of pp/dd.
#pragma unroll
      for (int k2 = 0; k2 < 2; k2++) {
        const int kq = 2 * mt + k2, o4 = 4 * k2;
        const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pp[o4], pp[o4 + 1], pp[o4 + 2], pp[o4 + 3]});
        const bf16x8 da = __builtin_bit_cast(bf16x8, u32x4{dd[o4], dd[o4 + 1], dd[o4 + 2], dd[o4 + 3]});
#pragma unroll
        for (int dt = 0; dt < NDT; dt++) {
          const int o1 = xslot(offT0, 32 * dt) + 16 * kq * D, o2 = xslot(offT1, 32 * dt) + 16 * kq * D;
          dv[dt] = mfma32(pa, lds_read_tr8(cdO + o1, cdO + o2), dv[dt]);
          dk[dt] = mfma32(da, lds_read_tr8(cQ + o1, cQ + o2), dk[dt]);
        }
      }
    }
    __syncthreads();  // dS'^T complete in LDS

    // dQ' (64 x D) = dS' (64 x 128 keys) K (128 keys x D).
    f32x16 dq[DQ_MT];
#pragma unroll
    for (int i = 0; i < DQ_MT; i++) dq[i] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < BN / 16; kk++) {
      const bf16x8 bk = lds_read_tr8(sK + offK0 + 16 * kk * D, sK + offK1 + 16 * kk * D);
#pragma unroll
      for (int i = 0; i < DQ_MT; i++) {
        const int m8 = 32 * (dq_mt0 + i);
        const bf16x8 as = lds_read_tr8(sdSt + xslot(offS0, m8) + 16 * kk * BM, sdSt + xslot(offS1, m8) + 16 * kk * BM);
        dq[i] = mfma32(as, bk, dq[i]);
      }
    }
    // Element j of dq[i] is query 32(dq_mt0+i) + 8(j/4) + 4hi + j%4, d = dq_d.
    const size_t blk_off = ((size_t)(b * S + m0) * Hq + h) * D;
    float* dst_base = ATOMIC ? p.dq_accum + blk_off : p.dq_part + (size_t)jb * nq + blk_off;
    if (m0 + BM <= S) {
      // Whole block in range: row offsets are wave-uniform (scalar) operands.
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(dst_base, (uint32_t)BM * row_bytes);
      const uint32_t rb = opaque(row_bytes);
#pragma unroll
      for (int i = 0; i < DQ_MT; i++)
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const uint32_t so = (uint32_t)(32 * (dq_mt0 + i) + 8 * (j >> 2) + (j & 3)) * rb;
          if (ATOMIC)
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(dq[i][j], rs, dq_voff, so, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dq[i][j]), rs, dq_voff, so, 0);
        }
    } else {
#pragma unroll
      for (int i = 0; i < DQ_MT; i++)
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const int qr = 32 * (dq_mt0 + i) + 8 * (j >> 2) + 4 * hi + (j & 3);
          if (m0 + qr < S) {
            float* a = dst_base + (size_t)qr * Hq * D + dq_d;
            if (ATOMIC)
              unsafeAtomicAdd(a, dq[i][j]);
            else
              *a = dq[i][j];
          }
        }
    }
  }

  // Epilogue: element j of lane l is key 32w + 8(j/4) + 4hi + j%4, d = 32dt + l32.
  const float inv_scale = 1.f / p.scale;
#pragma unroll
  for (int dt = 0; dt < NDT; dt++) {
    const int d = 32 * dt + l32;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int key = n0 + 32 * w + 8 * (j >> 2) + 4 * hi + (j & 3);
      if (key < S) {
        if (PARTIAL) {
          const size_t off = ((size_t)(b * S + key) * Hq + h) * D + d;
          p.dk_part[off] = dk[dt][j];
          p.dv_part[off] = dv[dt][j] * inv_scale;
        } else {
          const size_t off = ((size_t)(b * S + key) * Hkv + kvh) * D + d;
          p.dk[off] = to_bf16(dk[dt][j]);
          p.dv[off] = to_bf16(dv[dt][j] * inv_scale);
        }
      }
    }
  }
}

template <int D, bool CAUSAL, bool ATOMIC, bool PARTIAL>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  const int n_nblk = (p.S + kBN - 1) / kBN;
  const long long nwg = (long long)p.B * p.Hq * n_nblk;
  hipLaunchKernelGGL((bwd_kernel<D, CAUSAL, ATOMIC, PARTIAL>), dim3((unsigned)nwg), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  const bool part = p.G > 1;
  if (p.use_atomic)
    return part ? launch_bwd_t<D, CAUSAL, true, true>(p, stream) : launch_bwd_t<D, CAUSAL, true, false>(p, stream);
  return part ? launch_bwd_t<D, CAUSAL, false, true>(p, stream) : launch_bwd_t<D, CAUSAL, false, false>(p, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  if (p.D == 64) return p.causal ? launch_bwd_d<64, true>(p, stream) : launch_bwd_d<64, false>(p, stream);
  return p.causal ? launch_bwd_d<128, true>(p, stream) : launch_bwd_d<128, false>(p, stream);
}

}  // namespace mi355
