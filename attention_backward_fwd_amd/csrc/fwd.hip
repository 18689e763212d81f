// Forward of exact softmax attention on gfx950: O = softmax(scale Q K^T) V and
// the per-row log-sum-exp.
//
// The FlashAttention forward (flashattn_fwd in the TileLang #940 examples)
// streams key/value blocks past a resident query block with an online
// softmax.  This kernel does the same with the products transposed, so that
// every query row lives in one lane:
//
//   S^T (keys x queries) = K (keys x D) * Q^T        A = K from LDS, B = Q in registers
//   O^T (D x queries)   += V^T (D x keys) * P^T      A = V via transposing LDS reads,
//                                                     B = P^T straight from S^T's registers
//
// In the 32x32 MFMA result layout a lane holds one column (here: one query)
// and 16 rows (keys), so the running row max and row sum are in-lane
// reductions plus a single exchange between the two wavefront halves, and the
// rescale factor of the online softmax is a per-lane scalar.
//
// Workgroup: 4 waves x 32 queries = 128 queries; key/value tiles of 64 rows,
// double-buffered in LDS and filled by LDS-DMA buffer loads one tile ahead
// (one workgroup barrier per tile), whose per-lane offsets are computed once
// per kernel rather than per tile.  Scores stay fp32; P is rounded
// to bf16 only as an MFMA operand; O is written as bf16 (RNE) and LSE as fp32
// natural log including the scale.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mi355 {

namespace {

constexpr int kFwdBM = 128;
constexpr int kFwdBN = 64;

// The online softmax keeps a per-row reference maximum m and accumulates
// l = sum exp(s - m) and O = sum exp(s - m) v.  Any reference gives the same
// O / l, so m is only raised when a new score exceeds it by more than
// 2^kRescaleLog2 in exp2 units; until then every exponent stays below that
// bound (fp32 accumulators and bf16 P are unaffected) and the O rescale is
// skipped for the whole wavefront.
constexpr float kRescaleLog2 = 8.f;

// Two waves per SIMD: this also keeps the kernel within 256 VGPRs, so the
// MFMA accumulators live in VGPRs next to the softmax arithmetic.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fwd_kernel(FwdParams p) {
  constexpr int BM = kFwdBM, BN = kFwdBN;
  constexpr int NKS = D / 16;  // MFMA k-steps over the head dimension
  constexpr int NDT = D / 32;  // 32-row tiles of O^T
  constexpr int TK = BN * D;   // elements of one K or V tile

  // Separate LDS objects for the two buffers, so that the compiler can tell
  // the tile being loaded (LDS-DMA in flight) from the tile being read.
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TK];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TK];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TK];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[TK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (scalar)
  const int hi = lane >> 5, l32 = lane & 31, L = lane & 15, Gp = (lane >> 4) & 1;
  const int Hq = p.Hq, G = p.G, Hkv = p.Hkv;
  const int n_mblk = (p.S + BM - 1) / BM;

  // Tile order: each XCD gets a contiguous range of (batch, KV head) groups
  // (packed sequences: every eighth group, so that sequences of unequal
  // length load the XCDs evenly) and works through them two at a time (one
  // at a time for packed sequences), so the groups' K/V stay in its L2;
  // query blocks run heaviest-first under causal masking, with a group's
  // query heads side by side.
  const int nwg = gridDim.x, NG = p.B * Hkv;
  int t = blockIdx.x, x = 0, nx = 1, NGx = NG;
  if (NG % 8 == 0) {
    t = xcd_remap(blockIdx.x, nwg);
    const int per = nwg / 8;
    x = t / per;
    t -= x * per;
    nx = 8;
    NGx = NG / 8;
  }
  const int per_group = n_mblk * G;
  int grp, mbo, r;
  if (!p.cu && nx == 8 && NGx % 2 == 0) {
    // Dense problems: two groups at a time, their blocks interleaved
    // heaviest-first.  Group after group, the last group's heaviest block
    // would start near the end and run alone while the XCD's other CUs idle.
    const int pair = t / (2 * per_group), u = t % (2 * per_group);
    mbo = u / (2 * G);
    grp = x * NGx + 2 * pair + (u / G) % 2;
    r = u % G;
  } else {
    grp = p.cu ? (t / per_group) * nx + x : x * NGx + t / per_group;
    mbo = (t % per_group) / G;
    r = t % G;
  }
  const int b = __builtin_amdgcn_readfirstlane(grp / Hkv), kvh = __builtin_amdgcn_readfirstlane(grp % Hkv);
  const int h = __builtin_amdgcn_readfirstlane(kvh * G + r);
  // This sequence's query and key rows (packed sequences: their own
  // lengths; query blocks past the end have nothing to do).  Causal blocks
  // still run heaviest-first.  Query i sees key j iff j <= i + off.
  const SeqRows sr = seq_rows(p.cu, p.T, b, p.S);
  const SeqRows sk = seq_rows(p.cu ? p.cu_k : nullptr, p.Tk, b, p.Sk);
  const int S = __builtin_amdgcn_readfirstlane(sr.len), row0 = __builtin_amdgcn_readfirstlane(sr.base);
  const int Sk = __builtin_amdgcn_readfirstlane(sk.len), krow0 = __builtin_amdgcn_readfirstlane(sk.base);
  const int off = Sk - S;
  const int n_mblk_b = (S + BM - 1) / BM;
  const int mb = CAUSAL ? (n_mblk_b - 1 - mbo) : mbo;
  if (mb < 0 || mb >= n_mblk_b) return;

  const size_t qrs = (size_t)Hq * D, kvrs = (size_t)Hkv * D;
  const uint16_t* Qb = p.q + ((size_t)row0 * Hq + h) * D;
  const uint16_t* Kb = p.k + ((size_t)krow0 * Hkv + kvh) * D;
  const uint16_t* Vb = p.v + ((size_t)krow0 * Hkv + kvh) * D;

  const int q0 = mb * BM + 32 * w;  // first query of this wave
  const int qi = q0 + l32;          // this lane's query
  // Keys the block's queries can see; none (n_tiles = 0) leaves O = 0 and
  // LSE = -inf.
  const int n_end = CAUSAL ? max(0, min(Sk, mb * BM + BM + off)) : Sk;
  const int n_tiles = (n_end + BN - 1) / BN;

  // K and V tiles arrive by LDS-DMA buffer loads, 16 bytes per lane: row r
  // of the tile lands unpadded at LDS row r with its 16-byte slots swizzled
  // (swz), as the reads below expect.  Each wave issues NLD of the tile's
  // 1 KB instructions.  The per-lane byte offsets of a full tile are the same
  // for every tile and for K and V (same row stride), so they are computed
  // once; the last tile of a sequence reads its final row again for rows
  // past the end (those keys are masked).
  constexpr int CPR = D / 8, RPI = 64 / CPR;  // 16-byte slots per row, rows per instruction
  constexpr int NLD = (BN * D / 512) / 4;     // instructions per wave per tile
  const uint32_t rowb = (uint32_t)kvrs * 2u;  // bytes per key row
  uint32_t voff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; i++) {
    const int r = (w + 4 * i) * RPI + lane / CPR;
    voff[i] = (uint32_t)r * rowb + (uint32_t)(((lane % CPR) ^ swz<D>(r)) << 4);
  }
  auto load_kv = [&](const uint16_t* g, int row0, uint16_t* tile) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(g + (size_t)row0 * kvrs, (uint32_t)BN * rowb);
    if (row0 + BN <= Sk) {
#pragma unroll
      for (int i = 0; i < NLD; i++) {
        const uint32_t o = voff[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(tile + (w + 4 * i) * 512), 16, o, 0, 0, 0);
      }
    } else {
      const int last = Sk - 1 - row0;
#pragma unroll
      for (int i = 0; i < NLD; i++) {
        const int r = (w + 4 * i) * RPI + lane / CPR;
        const uint32_t o = (uint32_t)min(r, last) * rowb + (uint32_t)(((lane % CPR) ^ swz<D>(r)) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(tile + (w + 4 * i) * 512), 16, o, 0, 0, 0);
      }
    }
  };
  if (n_tiles > 0) {
    load_kv(Kb, 0, sK0);
    load_kv(Vb, 0, sV0);
  }

  bf16x8 qf[NKS];
  if (qi < S) {
    const uint16_t* qr = Qb + (size_t)qi * qrs + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < NKS; ks++) qf[ks] = *reinterpret_cast<const bf16x8*>(qr + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < NKS; ks++) qf[ks] = bf16x8{};
  }

  // Per-lane LDS element offsets (16-byte row reads of K; transposing reads
  // of V); the loop derives the rest with XORs and 16-row additions.
  const int offA0 = swz_off<D>(l32, 8 * hi);
  const int tcol = 16 * Gp + 4 * (L & 3);
  const int offV00 = swz_off<D>(4 * hi + (L >> 2), tcol);
  const int offV10 = swz_off<D>(4 * hi + (L >> 2) + 8, tcol);

  const float c = p.scale * kLog2e;
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; dt++) oacc[dt] = f32x16{};
  float m_i = -INFINITY, l_i = 0.f;

  // One key/value tile; BUF selects the LDS buffers it reads (the other
  // pair receives the next tile meanwhile).
  auto tile = [&](auto buf_tag, int it) {
    constexpr int BUF = decltype(buf_tag)::value;
    const uint16_t* cK = BUF ? sK1 : sK0;
    const uint16_t* cV = BUF ? sV1 : sV0;
    uint16_t* nK = BUF ? sK0 : sK1;
    uint16_t* nV = BUF ? sV0 : sV1;
    const int n0 = it * BN;
    wait_vmem();
    lds_barrier();  // tile it resident; every wave is done with tile it-1
    if (it + 1 < n_tiles) {
      load_kv(Kb, n0 + BN, nK);
      load_kv(Vb, n0 + BN, nV);
    }
    // A wave whose queries all precede the tile has nothing to do in it.
    if (CAUSAL && n0 > q0 + 31 + off) return;
    const int offA = opaque_v(offA0), offV0 = opaque_v(offV00), offV1 = opaque_v(offV10);

    // S^T (64 keys x 32 queries): element j of s[mt] is key
    // n0 + 32mt + 8(j/4) + 4hi + j%4, query qi.
    // Operands are read one k-step ahead of the products that use them.
    f32x16 s[2] = {f32x16{}, f32x16{}};
    bf16x8 k0 = lds_read_b128(cK + offA), k1 = lds_read_b128(cK + offA + 32 * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ks++) {
      bf16x8 n0v = k0, n1v = k1;
      if (ks + 1 < NKS) {
        n0v = lds_read_b128(cK + xslot(offA, 16 * (ks + 1)));
        n1v = lds_read_b128(cK + xslot(offA, 16 * (ks + 1)) + 32 * D);
      }
      s[0] = mfma32(k0, qf[ks], s[0]);
      s[1] = mfma32(k1, qf[ks], s[1]);
      k0 = n0v;
      k1 = n1v;
      __builtin_amdgcn_sched_barrier(0);
    }

    // Edge tiles (past the end, or crossing the causal diagonal): a key at
    // tile offset k is visible iff k <= lim.
    if ((n0 + BN > Sk) || (CAUSAL && n0 + BN - 1 > q0 + off)) {
      const int lim = (CAUSAL ? min(Sk - 1, qi + off) : Sk - 1) - n0 - 4 * hi;
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int j = 0; j < 16; j++)
          if (32 * mt + 8 * (j >> 2) + (j & 3) > lim) s[mt][j] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int j = 0; j < 16; j++) mx = fmaxf(mx, s[mt][j]);
    mx = xhalf_max(mx);
    const float m_cand = fmaxf(m_i, mx);
    const bool upd = (m_cand - m_i) * c > kRescaleLog2;  // true on the first visible tile
    const float m_new = upd ? m_cand : m_i;
    const float mc = (m_new == -INFINITY ? 0.f : m_new) * c;
    const float alpha = __builtin_amdgcn_exp2f(m_i * c - mc);
    float rs = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[mt][j], c, -mc));
        s[mt][j] = e;
        rs += e;
      }
    l_i = fmaf(l_i, alpha, rs);
    m_i = m_new;
    if (__builtin_amdgcn_ballot_w64(upd) != 0) {
#pragma unroll
      for (int dt = 0; dt < NDT; dt++) oacc[dt] *= alpha;
    }

    // P^T as the B operand: k-step kk covers keys 16kk.. of the tile, in the
    // order the S^T result layout holds them.
    bf16x8 pb[4];
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const int mt = kk >> 1, o8 = 8 * (kk & 1);
      pb[kk] = pack8(s[mt][o8 + 0], s[mt][o8 + 1], s[mt][o8 + 2], s[mt][o8 + 3], s[mt][o8 + 4],
                     s[mt][o8 + 5], s[mt][o8 + 6], s[mt][o8 + 7]);
    }
    // O^T += V^T P^T with V^T read by transposing LDS reads, one product
    // ahead.
    auto rd = [&](int it) {
      const int kk = it / NDT, dt = it % NDT;
      return lds_read_tr8(cV + xslot(offV0, 32 * dt) + 16 * kk * D, cV + xslot(offV1, 32 * dt) + 16 * kk * D);
    };
    bf16x8 a = rd(0);
#pragma unroll
    for (int it = 0; it < 4 * NDT; it++) {
      bf16x8 a1 = a;
      if (it + 1 < 4 * NDT) a1 = rd(it + 1);
      oacc[it % NDT] = mfma32(a, pb[it / NDT], oacc[it % NDT]);
      a = a1;
    }
  };
  for (int it = 0; it < n_tiles; it += 2) {
    tile(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_tiles) tile(std::integral_constant<int, 1>{}, it + 1);
  }

  const float l_tot = xhalf_sum(l_i);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qi < S) {
    uint16_t* orow = p.o + ((size_t)(row0 + qi) * Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int jg = 0; jg < 4; jg++) {
        const int d = 32 * dt + 8 * jg + 4 * hi;
        u32x2 v2 = {pack_bf16x2(oacc[dt][4 * jg] * inv, oacc[dt][4 * jg + 1] * inv),
                    pack_bf16x2(oacc[dt][4 * jg + 2] * inv, oacc[dt][4 * jg + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d) = v2;
      }
    // LSE rows: [B][Hq][S], or [Hq][T] for packed sequences.
    const size_t lrow = p.cu ? (size_t)h * p.T + row0 : (size_t)(b * Hq + h) * S;
    if (hi == 0) p.lse[lrow + qi] = m_i * p.scale + __builtin_amdgcn_logf(l_tot) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
  const int n_mblk = (p.S + kFwdBM - 1) / kFwdBM;
  const long long nwg = (long long)p.B * p.Hq * n_mblk;
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  if (p.D == 64) return p.causal ? launch_fwd_t<64, true>(p, stream) : launch_fwd_t<64, false>(p, stream);
  return p.causal ? launch_fwd_t<128, true>(p, stream) : launch_fwd_t<128, false>(p, stream);
}

}  // namespace mi355
