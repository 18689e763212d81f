// Backward of exact softmax attention on gfx950 (dQ, dK, dV).
//
// Decomposition as in the FlashAttention backward examples of TileLang #940
// (flashattn_bwd_atomic_add / flashattn_bwd_split): one workgroup owns a block
// of keys of one (batch, query head), keeps its dK/dV accumulators on chip
// for the whole sweep and walks the query blocks that see those keys.  Each
// of the 8 waves owns 32-key tiles of the block: one at D = 128 (256 keys per
// block), two at D = 64 (512 keys).  Per 32-query block the five tile
// contractions run on the matrix cores:
//
//   S  = Q K^T            A = Q (LDS, row reads)      B = K (LDS, row reads)
//   dP = dO V^T           A = dO (LDS, row reads)     B = V (registers)
//   dV += P^T dO          A = P^T (registers)         B = dO (LDS, transposing reads)
//   dK += dS^T Q          A = dS^T (registers)        B = Q (LDS, transposing reads)
//   dQ  = dS K            A = dS (LDS, transposing)   B = K (LDS, transposing reads)
//
// with P recomputed from the forward's LSE and dS = P o (dP - Delta).  The
// 32x32 MFMA result layout puts one key in each lane and 16 query rows in its
// registers; that is already the A-operand layout of P^T and dS^T for the dV
// and dK products, so those never leave registers.  dQ needs dS with queries
// in lanes, so dS^T goes through LDS; dQ (32 queries x D) is split over the
// waves: for D = 128 waves 0-3 (one per SIMD) each form a 32x32 tile, for
// D = 64 every wave a 16x16 tile.
//
// Why tall key blocks: every key block adds its dQ contribution once per
// query block, so the dQ traffic leaving the workgroups (fp32 atomics, or the
// split path's partials) is inversely proportional to the key-block height,
// and the fp32 atomic rate of the memory system, not the matrix cores, bounds
// a 128-key version.  The dK/dV accumulators of 256 keys at D = 128 (512 at
// D = 64) fill half of the register file; V lives in registers (it is only
// ever a B operand of dP), which leaves LDS for K, double-buffered Q/dO
// blocks and dS^T.  At D = 64 the two tiles of a wave run one after the
// other within a step, and the step's fixed costs (barrier, dQ emission)
// are shared by twice the keys.
//
// The softmax scale is folded into the exponent: the kernel forms
// P' = scale * P = exp2(S*scale*log2e - (LSE*log2e - log2(scale))), so that
// dS' = P' o (dP - Delta) = scale * dS is what both dQ and dK need; only dV
// is divided by the scale, once, at the end.
//
// Q and dO blocks are double-buffered in LDS and filled by LDS-DMA loads
// issued one block ahead; one workgroup barrier per query block, after which
// the dQ of the previous block is formed from its completed dS^T tile.
//
// dQ leaves the workgroup either as fp32 atomic adds into one accumulator
// (the page's atomic variant, with fp32 rather than bf16 atomics) or as a
// plain store into this key block's own fp32 partial slot, summed later in a
// fixed order by dq_sum_kernel (the split+sum variant): every partial element
// has exactly one writer, which makes that path bitwise deterministic.
//
// dK/dV never use atomics.  With one query head per KV head they are written
// as bf16 here.  With grouped-query attention a workgroup sweeps G / P query
// heads of its group one after the other (their dK/dV contributions add up
// in its accumulators) and writes one fp32 partial; the postprocess sums a
// group's P partials in a fixed order (P: bwd_gqa_parts()).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mi355 {

namespace {

// Cache policy of the split path's dQ partial stores: nontemporal (each
// 128-byte row piece of a store is whole, and the dQ sum reads it once).
constexpr int kStreamStore = 2;


constexpr int kBM = 32;  // queries per step
constexpr int kNW = 8;   // waves per workgroup

// dS'^T tile [block keys][32 queries] bf16, 64-byte rows.  The 8-byte chunk
// index of row r is XORed with fS(r) (bits 3, 2, 4 of r to chunk bits 2, 1,
// 0), which keeps both of its access patterns free of bank conflicts: the
// writes (32 consecutive keys, one chunk) and the transposing reads of the
// dQ product (keys 8g + e, g < 4, e < 4, four consecutive chunks).
__device__ __forceinline__ int dst_f(int row) {
  return (((row >> 3) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 4) & 1);
}
__device__ __forceinline__ int dst_off(int row, int col) {
  return row * kBM + ((((col >> 2) ^ dst_f(row)) << 2) | (col & 3));
}

// Two waves per SIMD: the kernel must fit 256 VGPRs, which also keeps every
// MFMA accumulator in VGPRs.
template <int D, bool CAUSAL, bool ATOMIC, bool PARTIAL>
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(2))) void bwd_kernel(BwdParams p) {
  // Keys per workgroup: KT tiles of 32 keys per wave (tile tt of wave w:
  // keys 256tt + 32w ..), one tile at D = 128, two at D = 64.
  constexpr int BN = bwd_block_n(D), BM = kBM, NW = kNW;
  constexpr int KT = BN / (32 * NW);
  static_assert(BN == 32 * NW * KT && (KT == 1 || KT == 2), "32-key tiles, one or two per wave");
  constexpr int TQ = BM * D;  // elements of one Q or dO block
  constexpr int NKS = D / 16, NDT = D / 32;
  // dQ tiles (16 queries x 16 d) per wave: D = 128 has 16 tiles (wave w
  // takes d columns 16w.. for both query halves), D = 64 has 8 (one each).
  constexpr int NQT = D / 64;

  // Separate LDS objects, so that the compiler can tell the block being
  // loaded (LDS-DMA in flight) from the block being read and does not wait
  // for the former before reading the latter.  The compiler places objects
  // of larger alignment first: the query-block tiles, dS'^T and the rows go
  // below 64 KB, where their addresses fit the LDS instructions' offset
  // field, and the K block above them.  The 1 KB alignment also lets the
  // swizzles be applied as XORs on whole LDS addresses.
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sQ0[TQ];
  __shared__ __attribute__((aligned(1024))) uint16_t sQ1[TQ];
  __shared__ __attribute__((aligned(1024))) uint16_t sdO0[TQ];
  __shared__ __attribute__((aligned(1024))) uint16_t sdO1[TQ];
  // dS'^T [key][query] (dst_off()), one per step parity: block i's tile is
  // written in step i and read by the dQ product in step i + 1.
  __shared__ __attribute__((aligned(1024))) uint16_t sdSt0[BN * BM];
  __shared__ __attribute__((aligned(1024))) uint16_t sdSt1[BN * BM];
  // Raw LSE and Delta rows of the query block (LDS-DMA, one per buffer; the
  // 64-lane load also fills the 32 entries past the block, unused).
  __shared__ __attribute__((aligned(1024))) float sL0[64];
  __shared__ __attribute__((aligned(1024))) float sL1[64];
  __shared__ __attribute__((aligned(1024))) float sD0[64];
  __shared__ __attribute__((aligned(1024))) float sD1[64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (scalar)
  const int hi = lane >> 5, l32 = lane & 31;
  const int Hq = p.Hq, G = p.G, Hkv = p.Hkv;
  const int n_nblk = (p.Sk + BN - 1) / BN;
  // The workgroup sweeps HPW query heads of its group, one after the other;
  // the group's NP = G / HPW head chunks each leave one dK/dV partial.
  const int HPW = p.hpw, NP = G / HPW;

  // Tile order: each XCD gets a contiguous range of (batch, KV head) groups
  // (packed sequences: every eighth group, so that sequences of unequal
  // length load the XCDs evenly) and works through them a few at a time
  // (their Q/dO rows stay in its L2); key
  // blocks run heaviest-first (block 0 sees every query under causal
  // masking) with a group's head chunks side by side.
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
  // (Integer division runs on the vector unit; readfirstlane returns the
  // results to scalar registers, where everything derived from them stays.)
  const int per_group = n_nblk * NP;
  int grp, jbv, r;
  // Each XCD takes CH groups at a time: as many as keep about 8 MB of
  // shared rows in flight (Q and dO rows of one group's query heads (bf16)), at least 2, a power of two dividing
  // the XCD's group count (none: one at a time).
  const long long gbytes = 4LL * p.S * D * G;
  int CH = 2;
  while (2 * CH <= NGx && 2LL * CH * gbytes <= (8LL << 20)) CH *= 2;
  while (CH > 1 && NGx % CH) CH >>= 1;
  // Workgroups that sweep several heads are few and long: then all of the
  // XCD's groups go side by side, so that its key blocks run heaviest-first
  // over all of them (longest-first list scheduling evens out the CUs; with
  // a few groups at a time the last ones' heavy blocks start late and run
  // alone).
  if (HPW > 1) CH = NGx;
  if (nx == 8 && CH > 1) {
    // Their key blocks interleaved heaviest-first: group after group, the
    // last group's heaviest block would start near the end and run alone
    // while the XCD's other CUs idle.
    const int chunk = t / (CH * per_group), u = t % (CH * per_group);
    jbv = u / (CH * NP);
    const int gl = CH * chunk + (u / NP) % CH;  // group within this XCD's share
    grp = p.cu ? gl * nx + x : x * NGx + gl;
    r = u % NP;
  } else {
    grp = p.cu ? (t / per_group) * nx + x : x * NGx + t / per_group;
    jbv = (t % per_group) / NP;
    r = t % NP;
  }
  const int jb = __builtin_amdgcn_readfirstlane(jbv);
  const int b = __builtin_amdgcn_readfirstlane(grp / Hkv), kvh = __builtin_amdgcn_readfirstlane(grp % Hkv);
  const int hc = __builtin_amdgcn_readfirstlane(r);                  // head chunk
  const int h = __builtin_amdgcn_readfirstlane(kvh * G + hc * HPW);  // its first query head
  const int n0 = jb * BN;
  // This sequence's query and key rows (packed sequences: their own
  // lengths; key blocks past the end have nothing to do).  Query i sees key
  // j iff j <= i + off under causal masking.
  const SeqRows sr = seq_rows(p.cu, p.T, b, p.S);
  const SeqRows sk = seq_rows(p.cu ? p.cu_k : nullptr, p.Tk, b, p.Sk);
  const int S = __builtin_amdgcn_readfirstlane(sr.len), row0 = __builtin_amdgcn_readfirstlane(sr.base);
  const int Sk = __builtin_amdgcn_readfirstlane(sk.len), krow0 = __builtin_amdgcn_readfirstlane(sk.base);
  const int off = Sk - S;
  if (n0 >= Sk) return;
  // Row-indexed tensors: [B][Hq][S], or [Hq][T] for packed sequences; head
  // h + hh starts hh * hstr rows after head h.
  const size_t hrow0 = p.cu ? (size_t)h * p.T + row0 : (size_t)(b * Hq + h) * S;
  const size_t hstr = p.cu ? (size_t)p.T : (size_t)S;

  const size_t qrs = (size_t)Hq * D, kvrs = (size_t)Hkv * D;
  const uint16_t* Qb = p.q + ((size_t)row0 * Hq + h) * D;
  const uint16_t* dOb = p.dout + ((size_t)row0 * Hq + h) * D;
  const uint16_t* Kb = p.k + ((size_t)krow0 * Hkv + kvh) * D;
  const uint16_t* Vb = p.v + ((size_t)krow0 * Hkv + kvh) * D;
  const float* lse_b = p.lse + hrow0;
  const float* dl_b = p.delta + hrow0;

  const float c = p.scale * kLog2e;
  const float lsc = p.log2_scale;
  // Query blocks that see a key of this block: from the one holding query
  // n0 - off on (causal); none when that is past the end (dK = dV = 0).
  const int m_begin = CAUSAL ? max(n0 - off, 0) / BM * BM : 0;
  const int n_steps = S > m_begin ? (S - m_begin + BM - 1) / BM : 0;
  const int n_tot = HPW * n_steps;  // steps over all the workgroup's heads

  // LSE and Delta of a query block land in LDS as raw fp32 rows (waves 0
  // and 1 each issue one 4-byte LDS-DMA load); rows past the end repeat the
  // last row and are masked below.
  auto load_rows = [&](int hh, int m0, float* l_dst, float* d_dst) {
    if (w == 0) row_load_async(lse_b + hh * hstr + m0, S - m0, l_dst, lane);
    if (w == 1) row_load_async(dl_b + hh * hstr + m0, S - m0, d_dst, lane);
  };
  // Key block (resident for the whole sweep) and the first Q/dO block.
  tile_load_async<D, BN, NW>(Kb, kvrs, n0, Sk, sK, w, lane);
  if (n_steps > 0) {
    tile_load_async<D, BM, NW>(Qb, qrs, m_begin, S, sQ0, w, lane);
    tile_load_async<D, BM, NW>(dOb, qrs, m_begin, S, sdO0, w, lane);
    load_rows(0, m_begin, sL0, sD0);
  }
  // This wave's keys: n0 + 32w + l32.  Its V rows are the B operand of dP
  // (lane l: V[key][16ks + 8hi .. +7]) and stay in registers; keys past the
  // end read the last row (their P is masked to zero).  The first step
  // waits for every load anyway; waiting here, before the loop, lets the
  // compiler see that V is ready inside it.
  bf16x8 vb[KT][NKS];
#pragma unroll
  for (int tt = 0; tt < KT; tt++) {
    const int key_l = n0 + 256 * tt + 32 * w + l32;
    const uint16_t* vrow = Vb + (size_t)min(key_l, Sk - 1) * kvrs + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < NKS; ks++) vb[tt][ks] = *reinterpret_cast<const bf16x8*>(vrow + 16 * ks);
  }
  wait_vmem();

  f32x16 dk[KT][NDT], dv[KT][NDT];
#pragma unroll
  for (int tt = 0; tt < KT; tt++)
#pragma unroll
    for (int dt = 0; dt < NDT; dt++) {
      dk[tt][dt] = f32x16{};
      dv[tt][dt] = f32x16{};
    }

  // dQ tiles.  D = 128: waves 0-3 each compute 32 queries x d columns
  // 32w .. 32w+31 as one 32x32 tile (one such wave per SIMD, so the matrix
  // work per SIMD stays even; each dS'^T and K element is read by fewer
  // waves than with 16x16 tiles).  D = 64: every wave computes one 16x16
  // tile, d columns 16dq_dt .., queries 16dq_qt0 ...
  constexpr bool DQ32 = (D == 128);
  constexpr int DQF4 = DQ32 ? 4 : NQT;  // f32x4 registers of dQ per lane
  const bool dq_wave = DQ32 ? (w < 4) : true;
  const int dq_dt = (D == 128) ? w : (w & 3);
  const int dq_qt0 = (D == 128) ? 0 : (w >> 2);
  // dQ accumulator and partials are head-major ([.., B, Hq, S, D]): the rows
  // of one query block are one contiguous run.  16x16 result element j of
  // lane l is query 16qt + 4(l/16) + j, d 16dq_dt + l%16.
  const uint32_t row_bytes = (uint32_t)D * 4u;
  const uint32_t dq_voff = DQ32 ? (uint32_t)(4 * (lane >> 5)) * row_bytes + (uint32_t)(32 * w + (lane & 31)) * 4u
                                : (uint32_t)(4 * (lane >> 4)) * row_bytes + (uint32_t)(16 * dq_dt + (lane & 15)) * 4u;
  const size_t nq = (size_t)(p.cu ? p.T : p.B * p.S) * Hq * D;  // elements of one split partial slot
  constexpr int NEMIT = 4 * DQF4;  // atomics / stores per dQ wave per block

  auto dq_rsrc = [&](int hh, int m0) {
    const size_t blk_off = (hrow0 + hh * hstr + m0) * D;
    float* dst_base = ATOMIC ? p.dq_accum + blk_off : p.dq_part + (size_t)jb * nq + blk_off;
    return buffer_rsrc(dst_base, (uint32_t)BM * row_bytes);
  };
  // Element e % 4 of register e / 4 (e < NEMIT) to the block's rows: row
  // 8(e/4) + 4(l/32) + e%4 of the 32x32 tile, or 16(dq_qt0 + e/4) + 4(l/16)
  // + e%4 of the 16x16 tiles.
  auto dq_emit = [&](const __amdgpu_buffer_rsrc_t& rs, const f32x4* v, int e) {
    const uint32_t rb = opaque(row_bytes);
    const int i = e >> 2, j = e & 3;
    const uint32_t so = (uint32_t)(DQ32 ? 8 * i + j : 16 * (dq_qt0 + i) + j) * rb;
    if (ATOMIC)
      __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v[i][j], rs, dq_voff, so, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[i][j]), rs, dq_voff, so, kStreamStore);
  };

  // dQ' (32 x D) = dS' (32 x BN keys) K (BN keys x D) of one block as
  // 16x16 tiles, from the dS'^T tile `sdSt`.  Operands are read one key
  // slice ahead of the products.
  auto dq_block32 = [&](const uint16_t* sdSt, f32x4* dq) {
    // 32x32x16 products over 16 slices of 16 keys; transposing reads of
    // dS'^T (rows = keys) and K, in the layout of the dV/dK B operands.
    const int ln = opaque_v(lane);
    const int lhi = ln >> 5, lL = ln & 15, tcol = 16 * ((ln >> 4) & 1) + 4 * (lL & 3);
    const uint32_t offK0 = 2 * swz_off<D>(8 * lhi + (lL >> 2), 32 * w + tcol);
    const uint32_t offK1 = 2 * swz_off<D>(8 * lhi + (lL >> 2) + 4, 32 * w + tcol);
    const uint32_t offS0 = 2 * dst_off(8 * lhi + (lL >> 2), tcol);
    const uint32_t offS1 = 2 * dst_off(8 * lhi + (lL >> 2) + 4, tcol);
    // A 16-row step flips bit 4 of the dS'^T row, which enters its swizzle
    // (dst_f): odd slices XOR the element offset with 4 (8 bytes).  The K
    // swizzle only sees the low 4 row bits.
    auto rd = [&](int kk, bf16x8& a, bf16x8& bk) {
      const uint32_t fx = 8u * (kk & 1);
      a = lds_tr8_at(sdSt, (offS0 ^ fx) + 32u * kk * BM, (offS1 ^ fx) + 32u * kk * BM);
      bk = lds_tr8_at(sK, offK0 + 32u * kk * D, offK1 + 32u * kk * D);
    };
    f32x16 acc = f32x16{};
    bf16x8 a, bk;
    rd(0, a, bk);
#pragma unroll
    for (int kk = 0; kk < BN / 16; kk++) {
      bf16x8 a1 = a, bk1 = bk;
      if (kk + 1 < BN / 16) rd(kk + 1, a1, bk1);
      acc = mfma32(a, bk, acc);
      a = a1;
      bk = bk1;
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) dq[i] = f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
  };
  auto dq_block = [&](const uint16_t* sdSt, f32x4* dq) {
    if constexpr (DQ32) {
      if (dq_wave) dq_block32(sdSt, dq);
      return;
    }
    const int ln = opaque_v(lane);
    const int lL = ln & 15, lg = lL >> 2, lc = lL & 3, lg4 = ln >> 4;  // e, c, group of the 16x16 layout
    const uint32_t offK0 = 2 * swz_off<D>(8 * lg4 + lg, 16 * dq_dt + 4 * lc);  // transposing reads of K
    const uint32_t offK1 = 2 * swz_off<D>(8 * lg4 + lg + 4, 16 * dq_dt + 4 * lc);
    const uint32_t offS0 = 2 * dst_off(8 * lg4 + lg, 16 * dq_qt0 + 4 * lc);    // ... of dS'^T
    const uint32_t offS1 = 2 * dst_off(8 * lg4 + lg + 4, 16 * dq_qt0 + 4 * lc);
#pragma unroll
    for (int i = 0; i < NQT; i++) dq[i] = f32x4{};
    auto rd_k = [&](int kk) { return lds_tr8_at(sK, offK0 + 64u * kk * D, offK1 + 64u * kk * D); };
    auto rd_s = [&](int kk, int i) {
      return lds_tr8_at(sdSt, (offS0 ^ (32u * i)) + 64u * kk * BM, (offS1 ^ (32u * i)) + 64u * kk * BM);
    };
    bf16x8 bk = rd_k(0), as[NQT];
#pragma unroll
    for (int i = 0; i < NQT; i++) as[i] = rd_s(0, i);
#pragma unroll
    for (int kk = 0; kk < BN / 32; kk++) {
      bf16x8 bk1 = bk, as1[NQT];
#pragma unroll
      for (int i = 0; i < NQT; i++) as1[i] = as[i];
      if (kk + 1 < BN / 32) {
        bk1 = rd_k(kk + 1);
#pragma unroll
        for (int i = 0; i < NQT; i++) as1[i] = rd_s(kk + 1, i);
      }
#pragma unroll
      for (int i = 0; i < NQT; i++) dq[i] = mfma16(as[i], bk, dq[i]);
      bk = bk1;
#pragma unroll
      for (int i = 0; i < NQT; i++) as[i] = as1[i];
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // dQ of the block at m0 of head h + hh leaves the workgroup: a full block
  // as buffer atomics/stores, the last, partial one row by row (addresses
  // derived here, not kept live).
  auto dq_store = [&](int hh, int m0, const f32x4* dq) {
    if (!dq_wave) return;
    if (m0 + BM <= S) {
      const __amdgpu_buffer_rsrc_t rs = dq_rsrc(hh, m0);
#pragma unroll
      for (int e = 0; e < NEMIT; e++) dq_emit(rs, dq, e);
    } else {
      const size_t blk_off = (hrow0 + hh * hstr + m0) * D;
      float* dst_base = ATOMIC ? p.dq_accum + blk_off : p.dq_part + (size_t)jb * nq + blk_off;
      const int lt = opaque_v(lane);
      const int tg = DQ32 ? lt >> 5 : lt >> 4;
      const int td = DQ32 ? 32 * w + (lt & 31) : 16 * dq_dt + (lt & 15);
#pragma unroll
      for (int i = 0; i < DQF4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int qr = DQ32 ? 8 * i + 4 * tg + j : 16 * (dq_qt0 + i) + 4 * tg + j;
          if (m0 + qr < S) {
            float* a = dst_base + (size_t)qr * D + td;
            if (ATOMIC)
              unsafeAtomicAdd(a, dq[i][j]);
            else
              *a = dq[i][j];
          }
        }
    }
  };

  // One query block; BUF selects the LDS buffers it reads (the other pair
  // receives the next block meanwhile) and the dS'^T tile it writes.  It
  // also computes and writes the dQ of the previous block from the other
  // dS'^T tile, completed by the barrier that starts this step.  Steps run
  // over the query blocks of head h, then those of h + 1, ...; cur_h and
  // cur_i name the head (from h) and query block of the current step.
  int cur_h = 0, cur_i = 0;
  auto step = [&](auto buf_tag, int st) {
    constexpr int BUF = decltype(buf_tag)::value;
    uint16_t* cQ = BUF ? sQ1 : sQ0;
    uint16_t* cdO = BUF ? sdO1 : sdO0;
    uint16_t* nQ = BUF ? sQ0 : sQ1;
    uint16_t* ndO = BUF ? sdO0 : sdO1;
    const float* cL = BUF ? sL1 : sL0;
    const float* cDl = BUF ? sD1 : sD0;
    float* nL = BUF ? sL0 : sL1;
    float* nD = BUF ? sD0 : sD1;
    uint16_t* wS = BUF ? sdSt1 : sdSt0;        // this block's dS'^T
    const uint16_t* pS = BUF ? sdSt0 : sdSt1;  // the previous block's
    const int hh = cur_h, m0 = m_begin + cur_i * BM;
    // The next block (loaded during this step) and the previous one (its dQ
    // leaves at the end of this step), across a change of head.
    const bool last_of_head = cur_i + 1 == n_steps;
    const int nh = last_of_head ? hh + 1 : hh, nm0 = last_of_head ? m_begin : m0 + BM;
    const int ph = cur_i == 0 ? hh - 1 : hh, pm0 = cur_i == 0 ? m_begin + (n_steps - 1) * BM : m0 - BM;
    // Block st resident.  From step 2 on, the dQ atomics/stores that ended
    // step st-1 (those of block st-2) came after those loads and may stay in
    // flight; step 0 wrote no dQ, so step 1 waits for everything.
    if (st > 1 && dq_wave)
      wait_vmem_but<NEMIT>();
    else
      wait_vmem();
    lds_barrier();  // block st resident, dS'^T of block st-1 complete; every wave is done with step st-1
    if (st + 1 < n_tot) {
      tile_load_async<D, BM, NW>(Qb + nh * D, qrs, nm0, S, nQ, w, lane);
      tile_load_async<D, BM, NW>(dOb + nh * D, qrs, nm0, S, ndO, w, lane);
      load_rows(nh, nm0, nL, nD);
    }
    // These loads stay ahead of this step's dQ atomics/stores in the
    // instruction stream: the next step's wait counts on that order.
    asm volatile("" ::: "memory");
    // Per-lane LDS byte offsets, recomputed from the lane id every step
    // rather than kept live across the loop; the loops below derive the rest
    // with XORs of column moves and additions of 16-row moves (see xslot()).
    const int ln = opaque_v(lane);
    const int lhi = ln >> 5, ll32 = ln & 31, lL = ln & 15, tcol = 16 * ((ln >> 4) & 1) + 4 * (lL & 3);
    const uint32_t offR = 2 * swz_off<D>(ll32, 8 * lhi);                // 16-byte row reads, row l32
    const uint32_t offT0 = 2 * swz_off<D>(4 * lhi + (lL >> 2), tcol);    // transposing reads of Q / dO
    const uint32_t offT1 = 2 * swz_off<D>(4 * lhi + (lL >> 2) + 8, tcol);

    // Keys n0 .. n0+n_vis-1 exist and see some query of this block.  A
    // 32-key tile of a wave past that has P = 0 throughout: it skips the four
    // products and writes zeros as its rows of dS'^T; the wave still takes
    // part in dQ and the barriers.
    // (Opaque per step: a loop-invariant value would let the compiler
    // specialise the loop body per tile state and spill.)
    const int n_vis = opaque(__builtin_amdgcn_readfirstlane(CAUSAL ? min(min(BN, Sk - n0), m0 + BM + off - n0)
                                                                   : min(BN, Sk - n0)));
    f32x4 dq[DQF4];
    // With two tiles the dQ product goes first, while only the accumulators
    // and V are live (between a tile's S/dP and its softmax there is no room).
    if (KT > 1 && st > 0) dq_block(pS, dq);
#pragma unroll
    for (int tt = 0; tt < KT; tt++) {
    const int kt0 = 256 * tt + 32 * w;  // first key of this tile in the block
    if (kt0 < n_vis) {
      // S = Q K^T and dP = dO V^T for the block's 32 queries x this tile's
      // 32 keys.  Operands are read one k-step ahead of the products that
      // use them.
      f32x16 s = f32x16{}, dp = f32x16{};
      {
        const uint16_t* kw_base = sK + kt0 * D;
        bf16x8 aq = lds_b128_at(cQ, offR), bk = lds_b128_at(kw_base, offR), ad = lds_b128_at(cdO, offR);
#pragma unroll
        for (int ks = 0; ks < NKS; ks++) {
          bf16x8 aq1 = aq, bk1 = bk, ad1 = ad;
          if (ks + 1 < NKS) {
            const uint32_t oq = offR ^ (32u * (ks + 1));
            aq1 = lds_b128_at(cQ, oq);
            bk1 = lds_b128_at(kw_base, oq);
            ad1 = lds_b128_at(cdO, oq);
          }
          s = mfma32(aq, bk, s);
          dp = mfma32(ad, vb[tt][ks], dp);
          aq = aq1;
          bk = bk1;
          ad = ad1;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (KT == 1 && st > 0) dq_block(pS, dq);

      // P' = scale P and dS' = scale dS.  Element j of lane l is query
      // 8(j/4) + 4hi + j%4 of the block, key kt0 + l32.
      const uint32_t orow = 16 * lhi;  // byte offset of query 4hi in the LSE / Delta rows
      uint32_t pp[8], dd[8];
      auto softmax_grad = [&](auto mask_tag, int qlim, int qend) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int jg = 0; jg < 4; jg++) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(cL) + orow + 32 * jg) *
                               kLog2e - lsc;
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(cDl) + orow + 32 * jg);
          float pv[4], dv4[4];
#pragma unroll
          for (int jj = 0; jj < 4; jj++) {
            const int j = 4 * jg + jj;
            float e = __builtin_amdgcn_exp2f(fmaf(s[j], c, -l4[jj]));
            if (MASK && (8 * jg + jj < qlim || 8 * jg + jj >= qend)) e = 0.f;
            pv[jj] = e;
            dv4[jj] = e * (dp[j] - d4[jj]);
          }
          pp[2 * jg] = pack_bf16x2(pv[0], pv[1]);
          pp[2 * jg + 1] = pack_bf16x2(pv[2], pv[3]);
          dd[2 * jg] = pack_bf16x2(dv4[0], dv4[1]);
          dd[2 * jg + 1] = pack_bf16x2(dv4[2], dv4[3]);
        }
      };
      // Tiles on the causal diagonal or at either end of the sequence are
      // masked.  This lane's key is hidden from block queries below qlim (all
      // of them for keys past the end, the earlier ones under causal masking)
      // and from queries at or past qend (rows past the end of the sequence);
      // both limits are taken relative to 4hi, so that the per-element query
      // index is a constant.
      if ((n0 + kt0 + 32 > Sk) || (m0 + BM > S) || (CAUSAL && m0 + off < n0 + kt0 + 32)) {
        const int key_e = n0 + kt0 + ll32;
        const int qlim = (key_e >= Sk ? BM : (CAUSAL ? key_e - off - m0 : -1)) - 4 * lhi;
        softmax_grad(std::true_type{}, qlim, S - m0 - 4 * lhi);
      } else {
        softmax_grad(std::false_type{}, 0, 0);
      }
      // dS'^T to LDS as [key][query]: four consecutive queries per 8-byte
      // write.
      {
        const uint32_t aW = lds_addr(wS) + 2 * dst_off(kt0 + ll32, 4 * lhi);
#pragma unroll
        for (int jg = 0; jg < 4; jg++) lds_store_b64_addr(aW ^ (16u * jg), u32x2{dd[2 * jg], dd[2 * jg + 1]});
      }
      // dV += P'^T dO and dK += dS'^T Q over the block's 32 queries; the B
      // operands are columns of dO and Q, fetched (one product ahead) with
      // transposing LDS reads in the query order of pp/dd.
      {
        auto tr_off = [&](int it, int which) {  // it = k2 * NDT + dt
          const int k2 = it / NDT, dt = it % NDT;
          return ((which ? offT1 : offT0) ^ (64u * dt)) + 32u * k2 * D;
        };
        bf16x8 bo = lds_tr8_at(cdO, tr_off(0, 0), tr_off(0, 1));
        bf16x8 bq = lds_tr8_at(cQ, tr_off(0, 0), tr_off(0, 1));
#pragma unroll
        for (int it = 0; it < 2 * NDT; it++) {
          bf16x8 bo1 = bo, bq1 = bq;
          if (it + 1 < 2 * NDT) {
            bo1 = lds_tr8_at(cdO, tr_off(it + 1, 0), tr_off(it + 1, 1));
            bq1 = lds_tr8_at(cQ, tr_off(it + 1, 0), tr_off(it + 1, 1));
          }
          const int o4 = 4 * (it / NDT), dt = it % NDT;
          const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pp[o4], pp[o4 + 1], pp[o4 + 2], pp[o4 + 3]});
          const bf16x8 da = __builtin_bit_cast(bf16x8, u32x4{dd[o4], dd[o4 + 1], dd[o4 + 2], dd[o4 + 3]});
          dv[tt][dt] = mfma32(pa, bo, dv[tt][dt]);
          dk[tt][dt] = mfma32(da, bq, dk[tt][dt]);
          bo = bo1;
          bq = bq1;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      if (KT == 1 && st > 0) dq_block(pS, dq);
      // Zero rows of dS'^T, so that the dQ product can run over all keys.
      const uint32_t aW = lds_addr(wS) + 2 * dst_off(kt0 + ll32, 4 * lhi);
#pragma unroll
      for (int jg = 0; jg < 4; jg++) lds_store_b64_addr(aW ^ (16u * jg), u32x2{0u, 0u});
    }
    // (Tiles one after the other: their live ranges must not overlap.)
    __builtin_amdgcn_sched_barrier(0);
    }
    if (st > 0) dq_store(ph, pm0, dq);
    cur_h = nh;
    cur_i = last_of_head ? 0 : cur_i + 1;
  };

  for (int st = 0; st < n_tot; st += 2) {
    step(std::integral_constant<int, 0>{}, st);
    if (st + 1 < n_tot) step(std::integral_constant<int, 1>{}, st + 1);
  }
  // dQ of the last block.
  if (n_tot > 0) {
    lds_barrier();  // its dS'^T complete
    f32x4 dq[DQF4];
    dq_block(((n_tot - 1) & 1) ? sdSt1 : sdSt0, dq);
    dq_store(HPW - 1, m_begin + (n_steps - 1) * BM, dq);
  }
  // Each wave holds the complete dK/dV of its KT tiles of 32 keys.  Element
  // j of lane l of tile (tt, dt) is key 256tt + 32w + 8(j/4) + 4hi + j%4,
  // d = 32dt + l32.
  const float inv_scale = 1.f / p.scale;
  const int le = opaque_v(lane);  // output addresses derived here, not kept live
  const int ehi = le >> 5, el32 = le & 31;
#pragma unroll
  for (int tt = 0; tt < KT; tt++)
#pragma unroll
    for (int dt = 0; dt < NDT; dt++) {
      const int d = 32 * dt + el32;
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int key = n0 + 256 * tt + 32 * w + 8 * (j >> 2) + 4 * ehi + (j & 3);
        if (key < Sk) {
          if (PARTIAL) {
            // Streaming stores: the group sum reads each partial once.
            const size_t o = ((size_t)(krow0 + key) * (Hkv * NP) + kvh * NP + hc) * D + d;
            __builtin_nontemporal_store(dk[tt][dt][j], p.dk_part + o);
            __builtin_nontemporal_store(dv[tt][dt][j] * inv_scale, p.dv_part + o);
          } else {
            const size_t o = ((size_t)(krow0 + key) * Hkv + kvh) * D + d;
            p.dk[o] = to_bf16(dk[tt][dt][j]);
            p.dv[o] = to_bf16(dv[tt][dt][j] * inv_scale);
          }
        }
      }
    }
}

template <int D, bool CAUSAL, bool ATOMIC, bool PARTIAL>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  const int n_nblk = (p.Sk + bwd_block_n(D) - 1) / bwd_block_n(D);
  const long long nwg = (long long)p.B * p.Hkv * (p.G / p.hpw) * n_nblk;
  hipLaunchKernelGGL((bwd_kernel<D, CAUSAL, ATOMIC, PARTIAL>), dim3((unsigned)nwg), dim3(kNW * 64), 0, stream, p);
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
