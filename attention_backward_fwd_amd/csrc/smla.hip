// Sparse MLA attention: each query token attends to the latent key rows its
// index list selects (top-k, -1 for an unused slot), the way the Megatron-LM
// pull request "TileLang implementation of the fused DSA operations" (NVIDIA
// Megatron-LM #5049, file table and review summary) adds it: 576-wide latent
// rows as keys, their first 512 channels as values, bf16 in, fp32
// accumulation.  Per token t and head h, over the valid entries i of idx[t]:
//   s_i = scale q[t,h] . kv[idx[t,i]],  P = softmax(s),  O = sum_i P_i kv[idx[t,i], :512]
//   LSE = log sum_i exp(s_i)  (O = 0, LSE = -inf without a valid entry)
//
// Forward kernel: one workgroup (4 waves) per (token, 32-head tile).  Per
// tile of 32 entries the key rows are gathered by LDS-DMA (one tile ahead)
// into five swizzled sub-tiles (four of 128 channels, one of 64).  Wave w
// owns heads h0 + 16(w & 1) .. +15 and entries 16(w >> 1) .. +15 of each
// tile and computes their scores S^T = KV Q^T over all 576 channels with
// 16x16x32 products (query operands in registers); the two waves sharing a
// head set swap their tile maxima through LDS (one common softmax reference
// per head, moved lazily) and their probabilities (each needs all 32
// entries for its 256 output channels O^T = V^T P^T, transposing reads).
// Tiles past the last valid entry of the list are skipped; tokens are dealt
// to the XCDs round-robin, longest lists first.
#include "common.h"
#include "kernels.h"
#include "smla_split.h"

namespace mi355 {

namespace {

constexpr int kQK = 576, kVD = 512;
constexpr int kHT = 32;  // heads per workgroup
constexpr int kKT = 32;  // entries per tile
constexpr int kSub = kKT * 128;  // elements of a 128-channel sub-tile of 32 rows
// Backward: the dKV atomics of a tile that may still be in flight when the
// next tile starts (each wave issues 64 or 80 per tile; the counter holds 63).
constexpr int kAtomSlack = 48;
// The same for the split backward's 16-byte partial-row stores (16 or 20 per
// wave and tile: four per channel block, each a distinct 16-byte piece, so no
// compilation can issue fewer; more would only make the wait stricter).
constexpr int kStoreSlack = 16;
// Byte offset past the end of any dKV accumulator (at most kSmlaMaxKvTokens
// rows of 576 fp32): atomics sent there are dropped.
constexpr uint32_t kDropOffset = 0x7FFFFFF0u;
static_assert((uint64_t)kSmlaMaxKvTokens * kQK * 4 < kDropOffset, "drop offset inside the accumulator");

// Element offset of (row, col) in the sub-tile layout of a [32][576] tile:
// sub-tile col / 128 (the last one 64 wide), each swizzled on its own.
__device__ __forceinline__ int sub_off(int row, int col) {
  const int st = col >> 7, c = col & 127;
  return st * kSub + (st < 4 ? swz_off<128>(row, c) : swz_off<64>(row, c));
}

// 32x32x16 operands (k order: lane half hi gets k = 4hi..4hi+3, 8+4hi..8+4hi+3
// of each 16-step, the row order of a 32x32 result's elements 0..7).
// Transposing: tile [k][x] with x inside one 128-channel sub-tile `st`.
__device__ __forceinline__ bf16x8 sop_tr(const uint16_t* t, int st, int k0, int x0, int lane) {
  const int hi = lane >> 5, L = lane & 15, gp = (lane >> 4) & 1;
  const int col = x0 + 16 * gp + 4 * (L & 3);
  const uint16_t* s = t + st * kSub;
  return lds_read_tr8(s + swz_off<128>(k0 + 4 * hi + (L >> 2), col), s + swz_off<128>(k0 + 8 + 4 * hi + (L >> 2), col));
}

// Transposing read from the 64-channel sub-tile (channels 512 .. 575).
__device__ __forceinline__ bf16x8 sop_tr64(const uint16_t* t, int k0, int x0, int lane) {
  const int hi = lane >> 5, L = lane & 15, gp = (lane >> 4) & 1;
  const int col = x0 + 16 * gp + 4 * (L & 3);
  const uint16_t* s = t + 4 * kSub;
  return lds_read_tr8(s + swz_off<64>(k0 + 4 * hi + (L >> 2), col), s + swz_off<64>(k0 + 8 + 4 * hi + (L >> 2), col));
}
// Entry lists.  Wave 0 copies the raw indices of tile it (entries
// 32it .. 32it+31, addresses clamped to the list) into an LDS slot by
// LDS-DMA; an entry is used iff it lies inside the list and 0 <= j < Tk.
__device__ __forceinline__ void load_entries_async(const int* idx_t, int it, int K, int* slot, int w, int lane) {
  if (w == 0 && lane < kKT) dma_b32_asm(idx_t + min(it * kKT + lane, K - 1), lds_addr(slot));
}
// The same for a second per-entry list (the split backward's partial-row
// positions), issued right after the index list.
__device__ __forceinline__ void load_entries2_async(const int* idx_t, const int* pos_t, int it, int K, int* slot,
                                                    int* pslot, int w, int lane) {
  load_entries_async(idx_t, it, K, slot, w, lane);
  if (pos_t) load_entries_async(pos_t, it, K, pslot, w, lane);
}
__device__ __forceinline__ bool entry_ok(const int* slot, int r, int e0, int K, int Tk) {
  const int j = slot[r];
  return e0 + r < K && j >= 0 && j < Tk;
}
__device__ __forceinline__ int entry_row(const int* slot, int r, int e0, int K, int Tk) {
  return entry_ok(slot, r, e0, K, Tk) ? slot[r] : 0;
}

// Gather the rows of tile entries r < 32 (unused entries: row 0) of a
// [*][576] bf16 matrix into a tile in the sub-tile layout, by LDS-DMA.  Per
// wave: 2 instructions per 128-channel sub-tile (rows 4w + lane/16 and
// 16 + 4w + lane/16, one 256-byte row piece per 16 lanes), 1 for the
// 64-channel one (rows 8w + lane/8), 9 in all.  `cb` and `cb64` are the
// lane's swizzled byte offsets inside the row pieces (gather_cols).
struct GatherCols {
  uint32_t cb, cb64;
};
__device__ __forceinline__ GatherCols gather_cols(int w, int lane) {
  const int r = 4 * w + (lane >> 4), r64 = 8 * w + (lane >> 3);
  return {(uint32_t)(((lane & 15) ^ swz<128>(r)) << 4), (uint32_t)(1024 + (((lane & 7) ^ swz<64>(r64)) << 4))};
}
__device__ __forceinline__ void gather_rows_async(const uint16_t* g, const int* slot, int e0, int K, int Tk,
                                                  uint16_t* tile, GatherCols gc, int w, int lane) {
  // The three rows of this lane (rows r and r + 16 share the swizzle).
  const int r = 4 * w + (lane >> 4);
  const char* gb = reinterpret_cast<const char*>(g);
  const char* p0 = gb + (size_t)entry_row(slot, r, e0, K, Tk) * (kQK * 2) + gc.cb;
  const char* p1 = gb + (size_t)entry_row(slot, r + 16, e0, K, Tk) * (kQK * 2) + gc.cb;
  const char* p2 = gb + (size_t)entry_row(slot, 8 * w + (lane >> 3), e0, K, Tk) * (kQK * 2) + gc.cb64;
  const uint32_t tb = lds_addr(tile);
  dma_b128_asm_off<0>(p0, tb + 2 * (w * 512));
  dma_b128_asm_off<0>(p1, tb + 2 * ((w + 4) * 512));
  dma_b128_asm_off<256>(p0, tb + 2 * (kSub + w * 512));
  dma_b128_asm_off<256>(p1, tb + 2 * (kSub + (w + 4) * 512));
  dma_b128_asm_off<512>(p0, tb + 2 * (2 * kSub + w * 512));
  dma_b128_asm_off<512>(p1, tb + 2 * (2 * kSub + (w + 4) * 512));
  dma_b128_asm_off<768>(p0, tb + 2 * (3 * kSub + w * 512));
  dma_b128_asm_off<768>(p1, tb + 2 * (3 * kSub + (w + 4) * 512));
  dma_b128_asm_off<0>(p2, tb + 2 * (4 * kSub + w * 512));
}

// Combine a per-lane value with the one held 16 lanes away (the other row of
// its pair of 16-lane rows): permlane16_swap(x, x) returns {own, other} in
// rows 0, 2 and {other, own} in rows 1, 3, so a symmetric operation of the
// pair is the result in every lane (VALU only, no LDS round trip).
__device__ __forceinline__ float x16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float x16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Number of 32-entry tiles up to and including the last valid entry of the
// list idx_t[0 .. K) (0 when it has none): tiles past it hold only unused
// slots and are skipped.  All 256 threads take part; `red` is 4 ints of LDS.
__device__ __forceinline__ int live_tiles(const int* idx_t, int K, int Tk, int* red, int w, int lane) {
  int last = -1;
  for (int e = threadIdx.x; e < K; e += 256) {
    const int j = idx_t[e];
    if (j >= 0 && j < Tk) last = e;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) last = max(last, __shfl_xor(last, off, 64));
  if (lane == 0) red[w] = last;
  lds_barrier();
  last = max(max(red[0], red[1]), max(red[2], red[3]));
  return __builtin_amdgcn_readfirstlane((last + kKT) / kKT);
}

// Forward kernel.  Two gather buffers (one tile ahead) keep the LDS at
// ~78 KB and the registers under 256, so that two workgroups share a CU.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void smla_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int* __restrict__ idx,
    uint16_t* __restrict__ o, float* __restrict__ lse, int T, int Tk, int H, int K, float scale) {
  constexpr int kTile = 4 * kSub + kKT * 64;
  __shared__ __attribute__((aligned(16))) uint16_t sKV[2 * kTile];
  __shared__ __attribute__((aligned(16))) int sIdx[3][kKT];
  __shared__ int sRed[4];
  __shared__ float sMx[4][64];
  __shared__ __attribute__((aligned(16))) u32x2 sPx[4][64];
  __shared__ float sL[4][64];

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int hh = w & 1, eh = w >> 1, partner = w ^ 2;
  const int n_ht = (H + kHT - 1) / kHT;
  const int id = blockIdx.x;
  const int t = __builtin_amdgcn_readfirstlane(T - 1 - id / n_ht), h0 = __builtin_amdgcn_readfirstlane((id % n_ht) * kHT);
  const int* idx_t = idx + (size_t)t * K;

  // Query operands (B of the 16x16x32 product, k = channel, n = head):
  // lane (head 16hh + r, group g) holds channels 32ks + 8g .. +7.
  bf16x8 bq[18];
  {
    const uint16_t* qr = q + ((size_t)t * H + min(h0 + 16 * hh + r, H - 1)) * kQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 18; ks++) bq[ks] = *reinterpret_cast<const bf16x8*>(qr + 32 * ks);
    // Complete these loads here, once: waits the compiler would otherwise
    // place at their first use inside the tile loop would run every tile
    // and drain the gathers in flight.
    asm volatile("s_waitcnt vmcnt(0)"
                 : "+v"(bq[0]), "+v"(bq[1]), "+v"(bq[2]), "+v"(bq[3]), "+v"(bq[4]), "+v"(bq[5]), "+v"(bq[6]),
                   "+v"(bq[7]), "+v"(bq[8]), "+v"(bq[9]), "+v"(bq[10]), "+v"(bq[11]), "+v"(bq[12]), "+v"(bq[13]),
                   "+v"(bq[14]), "+v"(bq[15]), "+v"(bq[16]), "+v"(bq[17]));
  }
  const int n_tiles = live_tiles(idx_t, K, Tk, sRed, w, lane);
  const GatherCols gcols = gather_cols(w, lane);
  if (n_tiles > 0) {
    load_entries_async(idx_t, 0, K, sIdx[0], w, lane);
    if (n_tiles > 1) load_entries_async(idx_t, 1, K, sIdx[1], w, lane);
    wait_vmem();
    lds_barrier();
    gather_rows_async(kv, sIdx[0], 0, K, Tk, sKV, gcols, w, lane);
  }
  // Per-lane byte offsets in a gathered tile.  S: row 16eh + r, channels
  // 32ks + 8g .. +7 (one 16-byte read).  O: V^T operand of channel block cb
  // (channels 256eh + 16cb ..), entries 4g .. 4g+3 and 16 + 4g .. (the
  // order of the probabilities: this wave's result rows for half eh, the
  // partner's for the other half), transposing reads.
  uint32_t offA[18], offV[16][2];
#pragma unroll
  for (int ks = 0; ks < 18; ks++) offA[ks] = 2u * (uint32_t)sub_off(16 * eh + r, 32 * ks + 8 * g);
#pragma unroll
  for (int cb = 0; cb < 16; cb++) {
    const int ch0 = 256 * eh + 16 * cb, st = ch0 >> 7, c = (ch0 & 127) + 4 * (r & 3);
    offV[cb][0] = 2u * (uint32_t)(st * kSub + swz_off<128>(4 * g + (r >> 2), c));
    offV[cb][1] = 2u * (uint32_t)(st * kSub + swz_off<128>(16 + 4 * g + (r >> 2), c));
  }

  const float c = scale * kLog2e;
  f32x4 oacc[16];
#pragma unroll
  for (int cb = 0; cb < 16; cb++) oacc[cb] = f32x4{};
  constexpr float kLazy = 8.f;
  float M = -INFINITY, l_i = 0.f;

  for (int it = 0; it < n_tiles; it++) {
    const uint16_t* cKV = sKV + (it & 1) * kTile;
    wait_vmem();
    lds_barrier();
    if (it + 2 < n_tiles) load_entries_async(idx_t, it + 2, K, sIdx[(it + 2) % 3], w, lane);
    if (it + 1 < n_tiles)
      gather_rows_async(kv, sIdx[(it + 1) % 3], (it + 1) * kKT, K, Tk, sKV + ((it + 1) & 1) * kTile, gcols, w, lane);
    const int* cl = sIdx[it % 3];
    const uint32_t vmask =
        (uint32_t)__builtin_amdgcn_ballot_w64(lane < kKT ? entry_ok(cl, lane, it * kKT, K, Tk) : false);
    f32x4 s;
    {
      // Operands fetched three k-steps ahead; two accumulation chains (even
      // and odd k-steps) added at the end.
      constexpr int PF = 4;
      bf16x8 ka[18];
      f32x4 s0 = f32x4{}, s1 = f32x4{};
#pragma unroll
      for (int i = 0; i < PF - 1; i++) ka[i] = lds_b128_at(cKV, offA[i]);
#pragma unroll
      for (int ks = 0; ks < 18; ks++) {
        if (ks + PF - 1 < 18) ka[ks + PF - 1] = lds_b128_at(cKV, offA[ks + PF - 1]);
        if (ks & 1)
          s1 = mfma16(ka[ks], bq[ks], s1);
        else
          s0 = mfma16(ka[ks], bq[ks], s0);
        __builtin_amdgcn_sched_barrier(0);
      }
      s = s0 + s1;
    }
    if (vmask != 0xFFFFFFFFu) {
      const uint32_t ml = vmask >> (16 * eh + 4 * g);
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (!((ml >> j) & 1u)) s[j] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = xhalf_max(x16_max(mx));
    sMx[w][lane] = mx;
    lds_barrier();
    const float mxc = fmaxf(mx, sMx[partner][lane]) * c;
    if (__builtin_amdgcn_ballot_w64(mxc > M + kLazy) != 0) {
      const float Mn = fmaxf(M, mxc);
      const float alpha = Mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(M - Mn);
      l_i *= alpha;
#pragma unroll
      for (int cb = 0; cb < 16; cb++) oacc[cb] *= alpha;
      M = Mn;
    }
    const float mc = M == -INFINITY ? 0.f : M;
    float e[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      e[j] = __builtin_amdgcn_exp2f(fmaf(s[j], c, -mc));
      l_i += e[j];
    }
    const u32x2 pw = u32x2{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3])};
    sPx[w][lane] = pw;
    lds_barrier();
    const u32x2 pp = sPx[partner][lane];
    const u32x2 p0 = eh ? pp : pw, p1 = eh ? pw : pp;
    const bf16x8 bp = __builtin_bit_cast(bf16x8, u32x4{p0[0], p0[1], p1[0], p1[1]});
#pragma unroll
    for (int cb = 0; cb < 16; cb++) oacc[cb] = mfma16(lds_tr8_at(cKV, offV[cb][0], offV[cb][1]), bp, oacc[cb]);
  }

  // Row sums: this wave's 16 entries (the four lane groups), then the
  // partner's (same reference).
  l_i = xhalf_sum(x16_sum(l_i));
  sL[w][lane] = l_i;
  lds_barrier();
  const float l_tot = eh ? sL[partner][lane] + l_i : l_i + sL[partner][lane];
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int h = h0 + 16 * hh + r;
  if (h < H) {
    uint16_t* orow = o + ((size_t)t * H + h) * kVD + 256 * eh + 4 * g;
#pragma unroll
    for (int cb = 0; cb < 16; cb++)
      *reinterpret_cast<u32x2*>(orow + 16 * cb) =
          u32x2{pack_bf16x2(oacc[cb][0] * inv, oacc[cb][1] * inv), pack_bf16x2(oacc[cb][2] * inv, oacc[cb][3] * inv)};
    if (eh == 0 && g == 0) lse[(size_t)t * H + h] = (M + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

// ------------------------------------------------------------ backward
// Preprocess: Delta[t,h] = sum_{d<512} O[t,h,d] dO[t,h,d] (one wave per row,
// 8 channels per lane); optionally zero the fp32 dKV accumulator.
__global__ __launch_bounds__(256) void smla_pre_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                       float* __restrict__ delta, float* __restrict__ dkv_acc,
                                                       long long rows, long long acc4) {
  const int lane = threadIdx.x & 63;
  for (long long r = ((long long)blockIdx.x * 256 + threadIdx.x) / 64; r < rows; r += (long long)gridDim.x * 4) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + (size_t)r * kVD + 8 * lane);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dout + (size_t)r * kVD + 8 * lane);
    float x = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      x = fmaf(__uint_as_float(a[i] << 16), __uint_as_float(b[i] << 16), x);
      x = fmaf(__uint_as_float(a[i] & 0xffff0000u), __uint_as_float(b[i] & 0xffff0000u), x);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    if (lane == 0) delta[r] = x;
  }
  if (dkv_acc)
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < acc4; i += (long long)gridDim.x * 256)
      reinterpret_cast<f32x4*>(dkv_acc)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Postprocess: dkv = bf16(dkv_acc), 8 values per thread.
__global__ __launch_bounds__(256) void smla_post_kernel(const float* __restrict__ acc, uint16_t* __restrict__ dkv,
                                                        long long n8) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long long)gridDim.x * 256) {
    const f32x4 a = reinterpret_cast<const f32x4*>(acc)[2 * i], b = reinterpret_cast<const f32x4*>(acc)[2 * i + 1];
    reinterpret_cast<u32x4*>(dkv)[i] = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                                              pack_bf16x2(b[2], b[3])};
  }
}

// Backward kernel: one workgroup (4 waves) per (token, 32-head tile).  Per
// tile of 32 entries (gathered as in the forward), wave w owns the block of
// entries 16(w >> 1) .. +15 and heads h0 + 16(w & 1) .. +15, as in the
// forward, and computes its scores S^T and dP^T = V dO^T over all channels
// with 16x16x32 products (the entries' rows from LDS, read once for both;
// the token's query and dO rows sit in LDS for the whole list, and every
// operand is read three k-steps ahead of its product): no partial sums
// cross waves.  Then
// P = exp(S - LSE), dS = P (dP - Delta) (padded heads and unused entries: 0),
// and the waves hand scale dS and P over through LDS as [entry][head] tiles
// (one barrier) for the two products that contract over entries or heads:
//   dQ^T += KV^T (scale dS)^T   (in registers across all tiles; wave w owns
//                                channel blocks w, w+4, .. of the 18 blocks of 32)
//   dKV   = (scale dS)^T Q + P^T dO   for the tile's 32 entries, same channel
//                                blocks, added to the fp32 accumulator row of
//                                each valid entry with buffer atomics that stay
//                                in flight into the next tile.
// dQ (bf16) is written at the end.  As in the forward, tokens are dealt to
// the XCDs round-robin and tiles past the last valid entry are skipped.  The
// atomic rate of the memory system (~340 G fp32 adds/s), not the matrix
// work, bounds this kernel: 576 adds per (token, valid entry).
// SPLIT: instead of the atomics, each valid entry's dKV row (this head
// tile's share) is stored whole as row pos[t, i] * n_ht + head tile of
// `part` (pos: the entry's place among the entries ordered by key row, then
// token, then slot); unused entries write row `dummy_row`, which nothing
// reads, so that every wave issues the same number of stores per tile.  The
// rows go out through a small per-wave LDS tile as streaming stores of whole
// 128-byte lines: with plain stores of the product's 32-byte pieces the
// caches fetched the lines being written and lost the gathered key rows
// (4.5 GB read per call instead of 1.0 GB).  A fixed-order sum over each key
// row's consecutive partial rows then gives dKV.
template <bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1))) void smla_bwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ dout,
    const int* __restrict__ idx, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dq, float* __restrict__ dkv_acc, float* __restrict__ part, const int* __restrict__ pos,
    long long dummy_row, int T, int Tk, int H, int K, float scale) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[4 * kSub + kKT * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sDO[4 * kSub];  // dout rows of the 32 heads
  __shared__ __attribute__((aligned(16))) uint16_t sKV0[4 * kSub + kKT * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sKV1[4 * kSub + kKT * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sDS[kKT * kHT];  // scale dS as [entry][head]
  __shared__ __attribute__((aligned(16))) uint16_t sPT[kKT * kHT];  // P as [entry][head]
  __shared__ __attribute__((aligned(16))) int sIdx[3][kKT];  // raw entry lists, as in the forward
  __shared__ __attribute__((aligned(16))) int sPos[SPLIT ? 3 : 1][kKT];  // SPLIT: partial-row positions
  // SPLIT: per wave, 16 entries x 32 channels of fp32 dKV^T regrouped so
  // that eight lanes hold one entry's 128-byte line.
  __shared__ __attribute__((aligned(16))) float sStage[SPLIT ? 4 : 1][SPLIT ? 16 * 32 : 4];
  __shared__ int sRed[4];

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), hi = lane >> 5;
  const int l32 = lane & 31, g = lane >> 4, r = lane & 15;
  const int hh = w & 1, eh = w >> 1;
  const int n_ht = (H + kHT - 1) / kHT;
  // Workgroups go to the XCDs round-robin, so consecutive ids spread a run
  // of tokens over all of them (list lengths, and so costs, change slowly
  // along the tokens); the last tokens, whose lists are usually the
  // longest, start first.
  const int id = blockIdx.x;
  const int t = __builtin_amdgcn_readfirstlane(T - 1 - id / n_ht), h0 = __builtin_amdgcn_readfirstlane((id % n_ht) * kHT);
  const int* idx_t = idx + (size_t)t * K;
  const int* pos_t = SPLIT ? pos + (size_t)t * K : nullptr;
  // This lane's head in the score block (result column r).
  const int hs = h0 + 16 * hh + r;
  const bool hs_ok = hs < H;
  const int hsc = min(hs, H - 1);
  const float lse_l2 = lse[(size_t)t * H + hsc] * kLog2e;  // -inf for a token without entries: P = 0 below
  const float dl = delta[(size_t)t * H + hsc];
  const float c = scale * kLog2e;

  {
    const uint16_t* qb = q + ((size_t)t * H) * kQK;
#pragma unroll
    for (int st = 0; st < 4; st++) tile_load_async<128, kHT, 4>(qb + 128 * st, kQK, h0, H, sQ + st * kSub, w, lane);
    tile_load_async<64, kHT, 4>(qb + 512, kQK, h0, H, sQ + 4 * kSub, w, lane);
  }
  const uint16_t* dob = dout + ((size_t)t * H) * kVD;
#pragma unroll
  for (int st = 0; st < 4; st++) tile_load_async<128, kHT, 4>(dob + 128 * st, kVD, h0, H, sDO + st * kSub, w, lane);
  // Score operands (B of the 16x16x32 product, k = channel, n = head hs):
  // lane (r, g) reads channels 32ks + 8g .. +7 of q[hs] from sQ and of
  // dout[hs] from sDO.
  // dKV's dO operand (A, k = head 16kk + op_k(i), m = channel 32 blk + l32)
  // for channel blocks w, w+4, w+8, w+12 (< 16).
  bf16x8 vdo[4][2];
#pragma unroll
  for (int bi = 0; bi < 4; bi++)
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
      const int ch = 32 * (w + 4 * bi) + l32;
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int h = min(h0 + 16 * kk + (i < 4 ? 4 * hi + i : 8 + 4 * hi + (i - 4)), H - 1);
        x[i] = from_bf16(dob[(size_t)h * kVD + ch]);
      }
      vdo[bi][kk] = pack8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
    }
  // Complete these loads here, once: waits the compiler would otherwise put
  // at their first use inside the tile loop would drain the gathers in flight.
  asm volatile("s_waitcnt vmcnt(0)"
               : "+v"(vdo[0][0]), "+v"(vdo[0][1]), "+v"(vdo[1][0]), "+v"(vdo[1][1]), "+v"(vdo[2][0]),
                 "+v"(vdo[2][1]), "+v"(vdo[3][0]), "+v"(vdo[3][1]));

  const int n_tiles = live_tiles(idx_t, K, Tk, sRed, w, lane);
  const GatherCols gcols = gather_cols(w, lane);
  // Entry lists and gathers as in the forward kernel.
  if (n_tiles > 0) {
    load_entries2_async(idx_t, pos_t, 0, K, sIdx[0], sPos[0], w, lane);
    if (n_tiles > 1) load_entries2_async(idx_t, pos_t, 1, K, sIdx[1], sPos[SPLIT ? 1 : 0], w, lane);
    wait_vmem();
    lds_barrier();
    gather_rows_async(kv, sIdx[0], 0, K, Tk, sKV0, gcols, w, lane);
  }
  // dKV accumulator as a buffer resource: an unused entry's atomics get an
  // offset past its end, which the hardware drops, so that every wave issues
  // the same number of atomics per tile whatever the entries (the wait at the
  // start of the next tile counts on that).
  const __amdgpu_buffer_rsrc_t acc_rs = buffer_rsrc(dkv_acc, (uint32_t)Tk * (uint32_t)(kQK * 4));
  // Byte offsets of the score block's operands, channels 32ks + 8g .. +7:
  // row 16eh + r of a gathered tile (A), row 16hh + r of sQ and sDO (B).
  // Inside a 128-channel sub-tile only ks % 4 changes the swizzled slot; the
  // sub-tile adds a constant.
  uint32_t offK[6], offH[6];
#pragma unroll
  for (int m = 0; m < 4; m++) {
    offK[m] = 2u * (uint32_t)swz_off<128>(16 * eh + r, 32 * m + 8 * g);
    offH[m] = 2u * (uint32_t)swz_off<128>(16 * hh + r, 32 * m + 8 * g);
  }
#pragma unroll
  for (int m = 0; m < 2; m++) {
    offK[4 + m] = 2u * (uint32_t)(4 * kSub + swz_off<64>(16 * eh + r, 32 * m + 8 * g));
    offH[4 + m] = 2u * (uint32_t)(4 * kSub + swz_off<64>(16 * hh + r, 32 * m + 8 * g));
  }
  auto sub_op = [&](const uint16_t* tl, const uint32_t(&o)[6], int ks) {
    return lds_b128_at(tl, ks < 16 ? o[ks & 3] + 2u * kSub * (ks >> 2) : o[ks - 12]);
  };
  // dQ's (scale dS)^T operand (B, k = entry, n = head l32), transposing reads
  // of the [entry][head] tile in the k order of sop_tr.
  const int gp = (lane >> 4) & 1, L = lane & 15;
  const uint32_t offD0 = 2u * (uint32_t)((4 * hi + (L >> 2)) * kHT + 16 * gp + 4 * (L & 3));

  const int nblk = w < 2 ? 5 : 4;  // channel blocks of this wave: w, w+4, w+8, w+12, (w+16)
  f32x16 dqa[5];
#pragma unroll
  for (int bi = 0; bi < 5; bi++) dqa[bi] = f32x16{};

  auto tile = [&](auto buf_tag, auto nb_tag, int it) {
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr int NB = decltype(nb_tag)::value;  // channel blocks of this wave
    const uint16_t* cKV = BUF ? sKV1 : sKV0;
    uint16_t* nKV = BUF ? sKV0 : sKV1;
    const int slot = it % 3;
    // Tile it resident.  It was gathered before the previous tile's dKV
    // atomics or stores (at least 16 per wave, issued after the gather),
    // which may stay in flight: the counter retires in issue order.
    if (it > 0)
      wait_vmem_but<SPLIT ? kStoreSlack : kAtomSlack>();
    else
      wait_vmem();
    lds_barrier();  // tile it and the list of tile it+1 resident; every wave is done with tile it-1
    if (it + 2 < n_tiles)
      load_entries2_async(idx_t, pos_t, it + 2, K, sIdx[(it + 2) % 3], sPos[SPLIT ? (it + 2) % 3 : 0], w, lane);
    if (it + 1 < n_tiles) gather_rows_async(kv, sIdx[(it + 1) % 3], (it + 1) * kKT, K, Tk, nKV, gcols, w, lane);
    const int* cIdx = sIdx[slot];
    const int e0 = it * kKT;
    const uint32_t vmask =
        (uint32_t)__builtin_amdgcn_ballot_w64(lane < kKT ? entry_ok(cIdx, lane, e0, K, Tk) : false);
    // SPLIT: the partial rows this lane stores: entry 16R + 8j + lane/8 for
    // round R and half j, 16 bytes (chunk lane % 8) of its 128-byte line per
    // channel block.
    float* trow[2][2] = {{nullptr, nullptr}, {nullptr, nullptr}};
    if constexpr (SPLIT) {
      // The four positions are read together (unconditionally: every slot
      // holds a value), then each row is chosen without branches; a
      // position outside [0, dummy_row) (none are) would store to the sink row.
      int pe[4];
#pragma unroll
      for (int q = 0; q < 4; q++) pe[q] = sPos[slot][8 * q + (lane >> 3)];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int et = 8 * q + (lane >> 3);
        const unsigned long long rv = (unsigned long long)(long long)pe[q] * (unsigned)n_ht + (unsigned)(h0 / kHT);
        const bool use = ((vmask >> et) & 1u) && rv < (unsigned long long)dummy_row;
        const unsigned long long rr = use ? rv : (unsigned long long)dummy_row;
        trow[q >> 1][q & 1] = part + rr * kQK + 4 * (lane & 7);
      }
    }
    // S^T and dP^T of the block: entries 16eh + 4g + j, head hs.
    f32x4 s = f32x4{}, dp = f32x4{};
    {
      // Operands fetched PF - 1 k-steps ahead of their products.
      constexpr int PF = 4;
      bf16x8 ka[18], qa[18], da[16];
      auto fetch = [&](int i) {
        ka[i] = sub_op(cKV, offK, i);
        qa[i] = sub_op(sQ, offH, i);
        if (i < 16) da[i] = sub_op(sDO, offH, i);
      };
#pragma unroll
      for (int i = 0; i < PF - 1; i++) fetch(i);
#pragma unroll
      for (int ks = 0; ks < 18; ks++) {
        if (ks + PF - 1 < 18) fetch(ks + PF - 1);
        s = mfma16(ka[ks], qa[ks], s);
        if (ks < 16) dp = mfma16(ka[ks], da[ks], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const uint32_t ml = vmask >> (16 * eh + 4 * g);
    float p[4], ds[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const bool ok = hs_ok && ((ml >> j) & 1u);
      p[j] = ok ? __builtin_amdgcn_exp2f(fmaf(s[j], c, -lse_l2)) : 0.f;
      ds[j] = p[j] * (dp[j] - dl);
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int e = 16 * eh + 4 * g + j;
      sDS[e * kHT + 16 * hh + r] = to_bf16(scale * ds[j]);
      sPT[e * kHT + 16 * hh + r] = to_bf16(p[j]);
    }
    lds_barrier();  // sDS / sPT complete
    // Per channel block of this wave: dQ^T += KV^T (scale dS)^T, and the
    // block's dKV (operands of the next block read while this one's products
    // run; the result leaves after the next block's products are issued).
    bf16x8 bds[2], ads[2], apt[2];
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
      bds[kk] = lds_tr8_at(sDS, offD0 + 2u * (16 * kk) * kHT, offD0 + 2u * (16 * kk + 8) * kHT);
      // (scale dS)^T and P^T rows of entry l32, heads in op_k order.
      const uint16_t* rd = sDS + l32 * kHT + 16 * kk;
      const uint16_t* rp = sPT + l32 * kHT + 16 * kk;
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(rd + 4 * hi), a1 = *reinterpret_cast<const u32x2*>(rd + 8 + 4 * hi);
      const u32x2 b0 = *reinterpret_cast<const u32x2*>(rp + 4 * hi), b1 = *reinterpret_cast<const u32x2*>(rp + 8 + 4 * hi);
      ads[kk] = __builtin_bit_cast(bf16x8, u32x4{a0[0], a0[1], a1[0], a1[1]});
      apt[kk] = __builtin_bit_cast(bf16x8, u32x4{b0[0], b0[1], b1[0], b1[1]});
    }
    // Operands of this wave's block bi (channel block w + 4 bi): in the
    // 128-channel sub-tile bi for bi < 4, else the 64-channel one (w < 2).
    // bi is a constant after unrolling, so no path is chosen at run time.
    auto blk_ops = [&](int bi, bf16x8(&o)[4]) {
      if (bi < 4) {
        o[0] = sop_tr(cKV, bi, 0, 32 * w, lane);
        o[1] = sop_tr(cKV, bi, 16, 32 * w, lane);
        o[2] = sop_tr(sQ, bi, 0, 32 * w, lane);
        o[3] = sop_tr(sQ, bi, 16, 32 * w, lane);
      } else {
        o[0] = sop_tr64(cKV, 0, 32 * w, lane);
        o[1] = sop_tr64(cKV, 16, 32 * w, lane);
        o[2] = sop_tr64(sQ, 0, 32 * w, lane);
        o[3] = sop_tr64(sQ, 16, 32 * w, lane);
      }
    };
    // SPLIT: dKV^T[channel][entry] (operands swapped), lane l32 holds entry
    // l32's channels 32 blk + c_row(j): four 16-byte pieces per block.
    // Atomic: dKV[entry][channel], lane l32 holds channel 32 blk + l32 of
    // entries c_row(j).
    auto emit = [&](int blk, const f32x16& acc) {
      if constexpr (SPLIT) {
        // Two rounds of 16 entries through this wave's staging tile (chunk c
        // of entry e at e * 32 + 4 (c ^ (e/2 % 8)) floats: both access
        // patterns spread over the banks); LDS operations of a wave run in
        // order, so each round's reads see its writes and precede the next
        // round's writes.  Every store then covers whole 128-byte lines, so
        // streaming stores do not leave partial lines to HBM.
        float* stg = sStage[w];
#pragma unroll
        for (int R = 0; R < 2; R++) {
          if ((l32 >> 4) == R) {
            const int e = l32 & 15;
#pragma unroll
            for (int gg = 0; gg < 4; gg++)
              *reinterpret_cast<f32x4*>(stg + e * 32 + 4 * ((2 * gg + hi) ^ ((e >> 1) & 7))) =
                  f32x4{acc[4 * gg], acc[4 * gg + 1], acc[4 * gg + 2], acc[4 * gg + 3]};
          }
          // Other lanes' writes feed these reads: keep the reads after the
          // (divergent) writes and executed by every lane.
          asm volatile("" ::: "memory");
          f32x4 v[2];
#pragma unroll
          for (int j = 0; j < 2; j++) {
            const int e = 8 * j + (lane >> 3);
            v[j] = *reinterpret_cast<const f32x4*>(stg + e * 32 + 4 * ((lane & 7) ^ ((e >> 1) & 7)));
          }
          asm volatile("" ::: "memory");  // ... and before the next round's writes
#pragma unroll
          for (int j = 0; j < 2; j++) __builtin_nontemporal_store(v[j], reinterpret_cast<f32x4*>(trow[R][j] + 32 * blk));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const int e = c_row(j, hi);
          const uint32_t off = ((vmask >> e) & 1u)
                                   ? (uint32_t)cIdx[e] * (uint32_t)(kQK * 4) + (uint32_t)(32 * blk + l32) * 4u
                                   : kDropOffset;
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[j], acc_rs, off, 0, 0);
        }
      }
    };
    bf16x8 op[2][4];
    f32x16 acc[2];
    blk_ops(0, op[0]);
#pragma unroll
    for (int bi = 0; bi < NB; bi++) {
      // Blocks w, w+4, w+8, w+12 (all with value channels), and w+16 for waves 0, 1.
      if (bi + 1 < NB) blk_ops(bi + 1, op[(bi + 1) & 1]);
      const bf16x8(&o)[4] = op[bi & 1];
      dqa[bi] = mfma32(o[0], bds[0], dqa[bi]);
      dqa[bi] = mfma32(o[1], bds[1], dqa[bi]);
      f32x16& a = acc[bi & 1];
      if constexpr (SPLIT) {
        a = mfma32(o[2], ads[0], f32x16{});
        a = mfma32(o[3], ads[1], a);
        if (bi < 4) {
          a = mfma32(vdo[bi][0], apt[0], a);
          a = mfma32(vdo[bi][1], apt[1], a);
        }
      } else {
        a = mfma32(ads[0], o[2], f32x16{});
        a = mfma32(ads[1], o[3], a);
        if (bi < 4) {
          a = mfma32(apt[0], vdo[bi][0], a);
          a = mfma32(apt[1], vdo[bi][1], a);
        }
      }
      if (bi > 0) emit(w + 4 * (bi - 1), acc[(bi - 1) & 1]);
    }
    emit(w + 4 * (NB - 1), acc[(NB - 1) & 1]);
  };
  // Waves 0, 1 own five channel blocks, waves 2, 3 four: one copy of the
  // loop each, so that block counts are constants inside it.
  auto run = [&](auto nb_tag) {
    for (int it = 0; it < n_tiles; it += 2) {
      tile(std::integral_constant<int, 0>{}, nb_tag, it);
      if (it + 1 < n_tiles) tile(std::integral_constant<int, 1>{}, nb_tag, it + 1);
    }
  };
  if (w < 2)
    run(std::integral_constant<int, 5>{});
  else
    run(std::integral_constant<int, 4>{});
  if (n_tiles == 0) wait_vmem();  // the query tile's loads

  // dq[t, head, channel]: dQ^T element j of block blk is channel
  // 32 blk + c_row(j), head h0 + l32; four consecutive channels per store.
  const int head = h0 + l32;
  if (head < H) {
    uint16_t* dqr = dq + ((size_t)t * H + head) * kQK;
#pragma unroll
    for (int bi = 0; bi < 5; bi++) {
      if (bi >= nblk) continue;
      const int blk = w + 4 * bi;
#pragma unroll
      for (int jg = 0; jg < 4; jg++)
        *reinterpret_cast<u32x2*>(dqr + 32 * blk + c_row(4 * jg, hi)) =
            u32x2{pack_bf16x2(dqa[bi][4 * jg], dqa[bi][4 * jg + 1]), pack_bf16x2(dqa[bi][4 * jg + 2], dqa[bi][4 * jg + 3])};
    }
  }
}

}  // namespace

hipError_t launch_smla_bwd_pre(const uint16_t* o, const uint16_t* dout, float* delta, float* dkv_acc, int T, int Tk,
                               int H, hipStream_t stream) {
  const long long rows = (long long)T * H, acc4 = dkv_acc ? (long long)Tk * kQK / 4 : 0;
  long long g = (rows + 3) / 4;
  if (acc4 / 256 > g) g = acc4 / 256;
  if (g > 256LL * 64) g = 256LL * 64;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(smla_pre_kernel, dim3((unsigned)g), dim3(256), 0, stream, o, dout, delta, dkv_acc, rows, acc4);
  return hipGetLastError();
}

hipError_t launch_smla_bwd(const uint16_t* q, const uint16_t* kv, const uint16_t* dout, const int* idx,
                           const float* lse, const float* delta, uint16_t* dq, float* dkv_acc, int T, int Tk, int H,
                           int K, float scale, hipStream_t stream) {
  const int n_ht = (H + kHT - 1) / kHT;
  hipLaunchKernelGGL(smla_bwd_kernel<false>, dim3((unsigned)((long long)T * n_ht)), dim3(256), 0, stream, q, kv, dout,
                     idx, lse, delta, dq, dkv_acc, nullptr, nullptr, 0LL, T, Tk, H, K, scale);
  return hipGetLastError();
}

hipError_t launch_smla_bwd_partial(const uint16_t* q, const uint16_t* kv, const uint16_t* dout, const int* idx,
                                   const float* lse, const float* delta, uint16_t* dq, float* part, const int* pos,
                                   int T, int Tk, int H, int K, float scale, hipStream_t stream) {
  const int n_ht = (H + kHT - 1) / kHT;
  const long long dummy_row = (long long)T * K * n_ht;
  hipLaunchKernelGGL(smla_bwd_kernel<true>, dim3((unsigned)((long long)T * n_ht)), dim3(256), 0, stream, q, kv, dout,
                     idx, lse, delta, dq, nullptr, part, pos, dummy_row, T, Tk, H, K, scale);
  return hipGetLastError();
}

hipError_t launch_smla_bwd_post(const float* dkv_acc, uint16_t* dkv, int Tk, hipStream_t stream) {
  const long long n8 = (long long)Tk * kQK / 8;
  long long g = (n8 + 255) / 256;
  if (g > 256LL * 64) g = 256LL * 64;
  hipLaunchKernelGGL(smla_post_kernel, dim3((unsigned)g), dim3(256), 0, stream, dkv_acc, dkv, n8);
  return hipGetLastError();
}

hipError_t launch_smla_fwd(const uint16_t* q, const uint16_t* kv, const int* idx, uint16_t* o, float* lse, int T,
                           int Tk, int H, int K, float scale, hipStream_t stream) {
  const int n_ht = (H + kHT - 1) / kHT;
  hipLaunchKernelGGL(smla_fwd_kernel, dim3((unsigned)((long long)T * n_ht)), dim3(256), 0, stream, q, kv, idx, o,
                     lse, T, Tk, H, K, scale);
  return hipGetLastError();
}

}  // namespace mi355
