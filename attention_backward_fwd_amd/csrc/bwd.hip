// Backward of exact softmax attention on gfx950 (dQ, dK, dV).
//
// Decomposition as in the FlashAttention backward examples of TileLang #940
// (flashattn_bwd_atomic_add / flashattn_bwd_split): one workgroup owns a block
// of 128 keys of one (batch, query head), keeps its dK/dV accumulators on
// chip for the whole sweep and walks the query blocks that see those keys.
// Per 64-query block the five tile contractions run on the matrix cores:
//
//   S  = Q K^T            A = Q (LDS, row reads)      B = K (registers)
//   dP = dO V^T           A = dO (LDS, row reads)     B = V (registers)
//   dV += P^T dO          A = P^T (registers)         B = dO (LDS, transposing reads)
//   dK += dS^T Q          A = dS^T (registers)        B = Q (LDS, transposing reads)
//   dQ  = dS K            A = dS (LDS, transposing)   B = K (LDS, transposing reads)
//
// with P = exp(S*scale - LSE) recomputed from the forward's LSE and
// dS = P o (dP - Delta).  The 32x32 MFMA result layout puts one key in each
// lane and 16 query rows in its registers; that is already the A-operand
// layout of P^T and dS^T for the dV and dK products, so those never leave
// registers.  dQ needs dS with queries in lanes, so dS^T goes through LDS.
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
#include "common.h"
#include "kernels.h"

namespace mi355 {

namespace {

constexpr int kBN = kBwdBlockN;  // keys per workgroup (4 waves x 32)
constexpr int kBM = 64;          // queries per step

template <int D, bool CAUSAL, bool ATOMIC, bool PARTIAL>
__global__ __launch_bounds__(256) void bwd_kernel(BwdParams p) {
  constexpr int BN = kBN, BM = kBM;
  constexpr int KP = D + 16;   // sK pitch (transposing reads)
  constexpr int QP = D + 8;    // sQ / sdO pitch (row and transposing reads)
  constexpr int SP = BM + 16;  // sdSt pitch: dS^T stored [key][query]
  constexpr int NKS = D / 16, NDT = D / 32, CH = D / 8;
  constexpr int QLD = BM * CH / 256;  // 16-byte chunks per thread per Q/dO block
  constexpr int KLD = BN * CH / 256;
  // dQ tile split over the 4 waves: D=128 -> one 32-wide d tile and both
  // 32-row query tiles per wave; D=64 -> one 32x32 tile per wave.
  constexpr int DQ_MT = (D == 128) ? 2 : 1;

  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sQ[BM * QP];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[BM * QP];
  __shared__ __attribute__((aligned(16))) uint16_t sdSt[BN * SP];
  __shared__ __attribute__((aligned(16))) float sL[BM];
  __shared__ __attribute__((aligned(16))) float sDl[BM];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hi = lane >> 5, l32 = lane & 31, L = lane & 15, Gp = (lane >> 4) & 1;
  const int S = p.S, Hq = p.Hq, G = p.G, Hkv = p.Hkv;
  const int n_nblk = (S + BN - 1) / BN;

  // Tile order: each XCD gets a contiguous range of (batch, KV head) groups;
  // inside it, key blocks run heaviest-first (block 0 sees every query under
  // causal masking), the group's query heads next to each other.
  const int nwg = gridDim.x, NG = p.B * Hkv;
  int t = blockIdx.x, x = 0, NGx = NG;
  if (NG % 8 == 0) {
    t = xcd_remap(blockIdx.x, nwg);
    const int per = nwg / 8;
    x = t / per;
    t -= x * per;
    NGx = NG / 8;
  }
  const int r = t % G;
  t /= G;
  const int grp = x * NGx + t % NGx;
  const int jb = t / NGx;
  const int b = grp / Hkv, kvh = grp % Hkv, h = kvh * G + r;
  const int n0 = jb * BN;

  const size_t qrs = (size_t)Hq * D, kvrs = (size_t)Hkv * D;
  const uint16_t* Qb = p.q + ((size_t)b * S * Hq + h) * D;
  const uint16_t* dOb = p.dout + ((size_t)b * S * Hq + h) * D;
  const uint16_t* Kb = p.k + ((size_t)b * S * Hkv + kvh) * D;
  const uint16_t* Vb = p.v + ((size_t)b * S * Hkv + kvh) * D;
  const float* lse_b = p.lse + (size_t)(b * Hq + h) * S;
  const float* dl_b = p.delta + (size_t)(b * Hq + h) * S;

  // This wave's 32 keys as MFMA B operands (K^T and V^T columns).
  const int key_l = n0 + 32 * w + l32;
  bf16x8 kf[NKS], vf[NKS];
  if (key_l < S) {
    const uint16_t* kr = Kb + (size_t)key_l * kvrs + 8 * hi;
    const uint16_t* vr = Vb + (size_t)key_l * kvrs + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < NKS; ks++) {
      kf[ks] = *reinterpret_cast<const bf16x8*>(kr + 16 * ks);
      vf[ks] = *reinterpret_cast<const bf16x8*>(vr + 16 * ks);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < NKS; ks++) {
      kf[ks] = bf16x8{};
      vf[ks] = bf16x8{};
    }
  }
  // The whole key block in LDS, for the dQ product.
#pragma unroll
  for (int i = 0; i < KLD; i++) {
    const int idx = tid + 256 * i, row = idx / CH, col = (idx % CH) * 8, key = n0 + row;
    u32x4 v4 = {0, 0, 0, 0};
    if (key < S) v4 = *reinterpret_cast<const u32x4*>(Kb + (size_t)key * kvrs + col);
    *reinterpret_cast<u32x4*>(&sK[row * KP + col]) = v4;
  }

  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; dt++) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }

  const float c = p.scale * kLog2e;
  const int m_begin = CAUSAL ? n0 : 0;  // n0 is a multiple of BM
  const int n_steps = (S - m_begin + BM - 1) / BM;

  u32x4 qr[QLD], dor[QLD];
  float lr = 0.f, dlr = 0.f;
  auto gload = [&](int m0) {
#pragma unroll
    for (int i = 0; i < QLD; i++) {
      const int idx = tid + 256 * i, row = idx / CH, col = (idx % CH) * 8, q = m0 + row;
      if (q < S) {
        qr[i] = *reinterpret_cast<const u32x4*>(Qb + (size_t)q * qrs + col);
        dor[i] = *reinterpret_cast<const u32x4*>(dOb + (size_t)q * qrs + col);
      } else {
        qr[i] = u32x4{0, 0, 0, 0};
        dor[i] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < BM) {
      const int q = m0 + tid;
      // Rows past the end get LSE = +inf, so P = 0 there without a mask.
      lr = q < S ? lse_b[q] * kLog2e : INFINITY;
      dlr = q < S ? dl_b[q] : 0.f;
    }
  };

  gload(m_begin);
  for (int st = 0; st < n_steps; st++) {
    const int m0 = m_begin + st * BM;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < QLD; i++) {
      const int idx = tid + 256 * i, row = idx / CH, col = (idx % CH) * 8;
      *reinterpret_cast<u32x4*>(&sQ[row * QP + col]) = qr[i];
      *reinterpret_cast<u32x4*>(&sdO[row * QP + col]) = dor[i];
    }
    if (tid < BM) {
      sL[tid] = lr;
      sDl[tid] = dlr;
    }
    __syncthreads();
    if (st + 1 < n_steps) gload(m0 + BM);

    // S = Q K^T and dP = dO V^T for 64 queries x this wave's 32 keys.
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < NKS; ks++) {
#pragma unroll
      for (int mt = 0; mt < 2; mt++) {
        const bf16x8 aq = lds_read_b128(&sQ[(32 * mt + l32) * QP + 16 * ks + 8 * hi]);
        s[mt] = mfma32(aq, kf[ks], s[mt]);
        const bf16x8 ad = lds_read_b128(&sdO[(32 * mt + l32) * QP + 16 * ks + 8 * hi]);
        dp[mt] = mfma32(ad, vf[ks], dp[mt]);
      }
    }

    // P = exp2(S*scale*log2e - LSE*log2e); dS = P (dP - Delta).  Element j of
    // lane l is query 32mt + 8(j/4) + 4hi + j%4, key 32w + l32.
    const bool need_mask = (n0 + BN > S) || (CAUSAL && m0 < n0 + BN);
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
#pragma unroll
      for (int jg = 0; jg < 4; jg++) {
        const int qo = 32 * mt + 8 * jg + 4 * hi;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[qo]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sDl[qo]);
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int j = 4 * jg + jj;
          float pv = __builtin_amdgcn_exp2f(fmaf(s[mt][j], c, -l4[jj]));
          if (need_mask) {
            const int q = m0 + qo + jj;
            if (key_l >= S || (CAUSAL && key_l > q)) pv = 0.f;
          }
          s[mt][j] = pv;
          dp[mt][j] = pv * (dp[mt][j] - d4[jj]);
        }
      }
    }

    // A operands (keys x queries) of the dV and dK products.
    bf16x8 pa[4], da[4];
#pragma unroll
    for (int kq = 0; kq < 4; kq++) {
      const int mt = kq >> 1, o8 = 8 * (kq & 1);
      pa[kq] = pack8(s[mt][o8 + 0], s[mt][o8 + 1], s[mt][o8 + 2], s[mt][o8 + 3], s[mt][o8 + 4],
                     s[mt][o8 + 5], s[mt][o8 + 6], s[mt][o8 + 7]);
      da[kq] = pack8(dp[mt][o8 + 0], dp[mt][o8 + 1], dp[mt][o8 + 2], dp[mt][o8 + 3], dp[mt][o8 + 4],
                     dp[mt][o8 + 5], dp[mt][o8 + 6], dp[mt][o8 + 7]);
    }

    // dS^T to LDS as [key][query]: four consecutive queries per 8-byte write.
    {
      uint16_t* dst = &sdSt[(32 * w + l32) * SP + 4 * hi];
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int jg = 0; jg < 4; jg++) {
          const int j = 4 * jg;
          u32x2 v2 = {pack_bf16x2(dp[mt][j], dp[mt][j + 1]), pack_bf16x2(dp[mt][j + 2], dp[mt][j + 3])};
          *reinterpret_cast<u32x2*>(dst + 32 * mt + 8 * jg) = v2;
        }
    }

    // dV += P^T dO and dK += dS^T Q; the B operands are columns of dO and Q,
    // fetched with transposing LDS reads in the query order of pa/da.
#pragma unroll
    for (int dt = 0; dt < NDT; dt++) {
      const int col = 32 * dt + 16 * Gp + 4 * (L & 3);
#pragma unroll
      for (int kq = 0; kq < 4; kq++) {
        const int row = 16 * kq + 4 * hi + (L >> 2);
        const bf16x8 bo = lds_read_tr8(&sdO[row * QP + col], &sdO[(row + 8) * QP + col]);
        dv[dt] = mfma32(pa[kq], bo, dv[dt]);
        const bf16x8 bq = lds_read_tr8(&sQ[row * QP + col], &sQ[(row + 8) * QP + col]);
        dk[dt] = mfma32(da[kq], bq, dk[dt]);
      }
    }
    __syncthreads();

    // dQ (64 x D) = dS (64 x 128 keys) K (128 keys x D).
    {
      const int nt = (D == 128) ? w : (w & 1);
      const int mt0 = (D == 128) ? 0 : (w >> 1);
      f32x16 dq[DQ_MT];
#pragma unroll
      for (int i = 0; i < DQ_MT; i++) dq[i] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < BN / 16; kk++) {
        const int krow = 16 * kk + 8 * hi + (L >> 2);
        const int kcol = 32 * nt + 16 * Gp + 4 * (L & 3);
        const bf16x8 bk = lds_read_tr8(&sK[krow * KP + kcol], &sK[(krow + 4) * KP + kcol]);
#pragma unroll
        for (int i = 0; i < DQ_MT; i++) {
          const int scol = 32 * (mt0 + i) + 16 * Gp + 4 * (L & 3);
          const bf16x8 as = lds_read_tr8(&sdSt[krow * SP + scol], &sdSt[(krow + 4) * SP + scol]);
          dq[i] = mfma32(as, bk, dq[i]);
        }
      }
      const int d = 32 * nt + l32;
#pragma unroll
      for (int i = 0; i < DQ_MT; i++) {
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const int q = m0 + 32 * (mt0 + i) + 8 * (j >> 2) + 4 * hi + (j & 3);
          if (q < S) {
            const size_t off = ((size_t)(b * S + q) * Hq + h) * D + d;
            const float val = dq[i][j] * p.scale;
            if (ATOMIC)
              unsafeAtomicAdd(p.dq_accum + off, val);
            else
              p.dq_part[(size_t)jb * ((size_t)p.B * S * Hq * D) + off] = val;
          }
        }
      }
    }
  }

  // Epilogue: element j of lane l is key 32w + 8(j/4) + 4hi + j%4, d = 32dt + l32.
#pragma unroll
  for (int dt = 0; dt < NDT; dt++) {
    const int d = 32 * dt + l32;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int key = n0 + 32 * w + 8 * (j >> 2) + 4 * hi + (j & 3);
      if (key < S) {
        if (PARTIAL) {
          const size_t off = ((size_t)(b * S + key) * Hq + h) * D + d;
          p.dk_part[off] = dk[dt][j] * p.scale;
          p.dv_part[off] = dv[dt][j];
        } else {
          const size_t off = ((size_t)(b * S + key) * Hkv + kvh) * D + d;
          p.dk[off] = to_bf16(dk[dt][j] * p.scale);
          p.dv[off] = to_bf16(dv[dt][j]);
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
