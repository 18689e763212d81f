// Deterministic dKV for the sparse MLA backward: per-entry partial rows and a
// fixed-order sum per key row, instead of fp32 atomics whose order (and so
// the last bits of dKV) changes from run to run.  The cuDNN frontend pull
// request "CSA: add fused Compressor forward+backward CuTe-DSL kernels
// (ported from Megatron-LM)" (NVIDIA cudnn-frontend #427, numerics and
// determinism section) treats an fp32-atomic accumulator as not
// deterministic and names a reduction of per-CTA partials in a fixed order
// as the deterministic alternative; the dense backward's split path does the
// same for dQ.
//
// With E = T * K entry slots (slot i of token t is entry e = t K + i; valid
// iff 0 <= idx[e] < Tk):
//   1. a stable LSD radix sort of the entries by key row (invalid entries
//      get key Tk and sort last), one or two passes of at most 10 bits:
//      per-tile digit counts, an exclusive scan of the counts in
//      digit-major order, then a stable scatter that ranks each tile's
//      items in order;
//   2. pos[e] = the entry's place in that order (written by the last
//      scatter), off[j] = the first place of key row j (off[Tk] = the
//      number of valid entries);
//   3. the backward kernel stores entry e's dKV row of head tile ht as
//      partial row pos[e] * n_ht + ht (one per entry and head tile, fp32);
//   4. dkv[j] = bf16 of the sum of partial rows off[j] n_ht .. off[j+1] n_ht - 1,
//      taken in one fixed order (below), 0 for a row no entry names.
// The order of every addition is a function of idx alone, so dKV is bitwise
// reproducible.
#include "common.h"
#include "kernels.h"
#include "smla_split.h"

namespace mi355 {

namespace {

constexpr int kQK = 576;
constexpr int kHT = 32;                   // heads per backward workgroup
constexpr int kSortThreads = 256;
constexpr int kSortRounds = 16;
constexpr int kSortTile = kSortThreads * kSortRounds;  // items per sort workgroup
constexpr int kMaxDigitBits = 10;
constexpr int kScanBlock = 4096;          // elements per scan workgroup (256 threads x 16)

__device__ __forceinline__ int entry_key(const int* idx, long long e, int Tk) {
  const int j = idx[e];
  return (j >= 0 && j < Tk) ? j : Tk;
}

// Digit counts of one tile of items (keys from `keys`, or from idx on the
// first pass): hist[d * n_tiles + tile].
__global__ __launch_bounds__(kSortThreads) void sort_hist_kernel(const int* __restrict__ keys,
                                                                 const int* __restrict__ idx, int Tk, long long n,
                                                                 int shift, int bits, int n_tiles,
                                                                 int* __restrict__ hist) {
  __shared__ int cnt[1 << kMaxDigitBits];
  const int nd = 1 << bits, tile = blockIdx.x;
  for (int d = threadIdx.x; d < nd; d += kSortThreads) cnt[d] = 0;
  __syncthreads();
  const long long base = (long long)tile * kSortTile;
  for (int r = 0; r < kSortRounds; r++) {
    const long long i = base + r * kSortThreads + threadIdx.x;
    if (i < n) {
      const int k = keys ? keys[i] : entry_key(idx, i, Tk);
      atomicAdd(&cnt[(k >> shift) & (nd - 1)], 1);
    }
  }
  __syncthreads();
  for (int d = threadIdx.x; d < nd; d += kSortThreads) hist[(long long)d * n_tiles + tile] = cnt[d];
}

// Exclusive scan of the 256 values of a workgroup (one per thread); `tot`
// gets the total.  `red` holds 4 ints.
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int* tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[w] = x;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; i++) before += red[i];
  if (tot) *tot = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return before + x - v;
}

// Exclusive scan of n int32 values (three launches): per-block sums, one
// workgroup scanning the block sums, then each block scanned with its offset.
__global__ __launch_bounds__(256) void scan_sums_kernel(const int* __restrict__ x, long long n, int* __restrict__ sums) {
  __shared__ int red[4];
  const long long b = (long long)blockIdx.x * kScanBlock + threadIdx.x * 16;
  int s = 0;
  for (int k = 0; k < 16; k++)
    if (b + k < n) s += x[b + k];
  int tot;
  block_exclusive_scan(s, red, &tot);
  if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

__global__ __launch_bounds__(1024) void scan_top_kernel(int* __restrict__ sums, int nb) {
  __shared__ int part[1024];
  const int per = (nb + 1023) / 1024, a = threadIdx.x * per, e = min(a + per, nb);
  int s = 0;
  for (int i = a; i < e; i++) s += sums[i];
  part[threadIdx.x] = s;
  __syncthreads();
  // Hillis-Steele over the 1024 thread totals (inclusive), in place.
  for (int o = 1; o < 1024; o <<= 1) {
    const int y = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += y;
    __syncthreads();
  }
  int run = part[threadIdx.x] - s;
  for (int i = a; i < e; i++) {
    const int v = sums[i];
    sums[i] = run;
    run += v;
  }
}

__global__ __launch_bounds__(256) void scan_apply_kernel(int* __restrict__ x, long long n,
                                                         const int* __restrict__ sums) {
  __shared__ int red[4];
  const long long b = (long long)blockIdx.x * kScanBlock + threadIdx.x * 16;
  int v[16], s = 0;
#pragma unroll
  for (int k = 0; k < 16; k++) {
    v[k] = b + k < n ? x[b + k] : 0;
    s += v[k];
  }
  int run = sums[blockIdx.x] + block_exclusive_scan(s, red, nullptr);
#pragma unroll
  for (int k = 0; k < 16; k++)
    if (b + k < n) {
      x[b + k] = run;
      run += v[k];
    }
}

// Stable scatter of one tile: items in tile order (round r, thread tid is
// item r * 256 + tid) go to offs[d * n_tiles + tile] + their rank among the
// tile's items of digit d.  Within a round a wave ranks its lanes of equal
// digit with ballots (one per digit bit); waves before it add their counts
// of that digit; `run` carries the counts of the earlier rounds.  On the
// last pass (pos given) the entry numbers are not written out: each valid
// entry's final place goes to pos[entry] instead.
__global__ __launch_bounds__(kSortThreads) void sort_scatter_kernel(
    const int* __restrict__ keys, const int* __restrict__ vals, const int* __restrict__ idx, int Tk, long long n,
    int shift, int bits, int n_tiles, const int* __restrict__ offs, int* __restrict__ okeys,
    int* __restrict__ ovals, int* __restrict__ pos) {
  __shared__ int run[1 << kMaxDigitBits];
  __shared__ int wc[4][1 << kMaxDigitBits];
  const int nd = 1 << bits, tile = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int d = threadIdx.x; d < nd; d += kSortThreads) {
    run[d] = offs[(long long)d * n_tiles + tile];
    wc[0][d] = wc[1][d] = wc[2][d] = wc[3][d] = 0;
  }
  __syncthreads();
  const unsigned long long below_mask = (1ull << lane) - 1ull;
  const long long base = (long long)tile * kSortTile;
  for (int r = 0; r < kSortRounds; r++) {
    const long long i = base + r * kSortThreads + threadIdx.x;
    const bool ok = i < n;
    int k = 0, v = 0;
    if (ok) {
      k = keys ? keys[i] : entry_key(idx, i, Tk);
      v = vals ? vals[i] : (int)i;
    }
    const int d = (k >> shift) & (nd - 1);
    unsigned long long same = __ballot(ok);
    for (int b = 0; b < bits; b++) {
      const bool bit = (d >> b) & 1;
      const unsigned long long m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int below = __popcll(same & below_mask);
    if (ok && below == 0) wc[w][d] = __popcll(same);
    __syncthreads();
    if (ok) {
      int rank = run[d] + below;
      for (int ww = 0; ww < w; ww++) rank += wc[ww][d];
      if ((unsigned)rank < (unsigned long long)n) {  // always: the counts cover the tile's items
        okeys[rank] = k;
        if (!pos)
          ovals[rank] = v;
        else if (k < Tk)
          pos[v] = rank;  // v < n: an entry number
      }
    }
    __syncthreads();
    for (int dd = threadIdx.x; dd < nd; dd += kSortThreads) {
      run[dd] += wc[0][dd] + wc[1][dd] + wc[2][dd] + wc[3][dd];
      wc[0][dd] = wc[1][dd] = wc[2][dd] = wc[3][dd] = 0;
    }
    __syncthreads();
  }
}

// off[j] = number of sorted keys below j, for j = 0 .. Tk (binary search).
__global__ __launch_bounds__(256) void row_offsets_kernel(const int* __restrict__ keys, long long n, int Tk,
                                                          int* __restrict__ off) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j > Tk) return;
  long long lo = 0, hi = n;
  while (lo < hi) {
    const long long mid = (lo + hi) >> 1;
    if (keys[mid] < j)
      lo = mid + 1;
    else
      hi = mid;
  }
  off[j] = (int)lo;
}

// dkv[j] from its partial rows R = off[j] n_ht .. off[j+1] n_ht - 1: thread
// group g (144 threads, four channels each) sums rows R0 + g, R0 + g + 4, ..
// in ascending order; the four group sums are then added as
// ((s0 + s1) + s2) + s3.  The order depends on the row count alone.
constexpr int kSumGroups = 4, kSumCols = kQK / 4;
__global__ __launch_bounds__(kSumGroups * kSumCols) void dkv_sum_kernel(const float* __restrict__ part,
                                                                        const int* __restrict__ off, long long n,
                                                                        int n_ht, uint16_t* __restrict__ dkv) {
  __shared__ f32x4 red[kSumGroups - 1][kSumCols];
  const int j = blockIdx.x, g = threadIdx.x / kSumCols, c4 = threadIdx.x % kSumCols;
  // Offsets are ascending and at most n; clamped all the same.
  const long long a = min(max((long long)off[j], 0LL), n), b = min(max((long long)off[j + 1], a), n);
  const long long r0 = a * n_ht, r1 = b * n_ht;
  const f32x4* p = reinterpret_cast<const f32x4*>(part) + c4;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  long long r = r0 + g;
  // Streaming loads: each partial row is read once.
  auto ld = [&](long long rr) { return __builtin_nontemporal_load(p + rr * kSumCols); };
  for (; r + 3 * kSumGroups < r1; r += 4 * kSumGroups) {
    const f32x4 a0 = ld(r), a1 = ld(r + kSumGroups), a2 = ld(r + 2 * kSumGroups), a3 = ld(r + 3 * kSumGroups);
    acc += a0;
    acc += a1;
    acc += a2;
    acc += a3;
  }
  for (; r < r1; r += kSumGroups) acc += ld(r);
  if (g > 0) red[g - 1][c4] = acc;
  __syncthreads();
  if (g == 0) {
    acc += red[0][c4];
    acc += red[1][c4];
    acc += red[2][c4];
    *reinterpret_cast<u32x2*>(dkv + (size_t)j * kQK + 4 * c4) = u32x2{pack_bf16x2(acc[0], acc[1]),
                                                                      pack_bf16x2(acc[2], acc[3])};
  }
}
static_assert(kSumGroups == 4, "the group sums are combined as four terms");

struct SplitLayout {
  size_t part, pos, off, k0, v0, k1, v1, hist, sums, total;
  long long n, hist_n;
  int n_tiles, n_scan_blocks, n_pass, bits0, bits1, n_ht;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

SplitLayout split_layout(int T, int Tk, int H, int K) {
  SplitLayout L{};
  L.n = (long long)T * K;
  L.n_ht = (H + kHT - 1) / kHT;
  L.n_tiles = (int)((L.n + kSortTile - 1) / kSortTile);
  const int bits = 32 - __builtin_clz((unsigned)Tk);  // keys 0 .. Tk
  L.n_pass = bits <= kMaxDigitBits ? 1 : 2;
  L.bits0 = (bits + L.n_pass - 1) / L.n_pass;
  L.bits1 = bits - L.bits0;
  L.hist_n = ((long long)1 << L.bits0) * L.n_tiles;
  L.n_scan_blocks = (int)((L.hist_n + kScanBlock - 1) / kScanBlock);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  L.part = take(((size_t)L.n * L.n_ht + 1) * kQK * sizeof(float));
  L.pos = take((size_t)L.n * 4);
  L.off = take(((size_t)Tk + 1) * 4);
  L.k0 = take((size_t)L.n * 4);
  L.v0 = take((size_t)L.n * 4);
  L.k1 = take((size_t)L.n * 4);
  L.v1 = take((size_t)L.n * 4);
  L.hist = take((size_t)L.hist_n * 4);
  L.sums = take((size_t)L.n_scan_blocks * 4);
  L.total = o;
  return L;
}

hipError_t launch_scan(int* x, long long n, int* sums, int nb, hipStream_t stream) {
  hipLaunchKernelGGL(scan_sums_kernel, dim3(nb), dim3(256), 0, stream, x, n, sums);
  hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(1024), 0, stream, sums, nb);
  hipLaunchKernelGGL(scan_apply_kernel, dim3(nb), dim3(256), 0, stream, x, n, sums);
  return hipGetLastError();
}

}  // namespace

size_t smla_split_workspace_bytes(int T, int Tk, int H, int K) { return split_layout(T, Tk, H, K).total; }

hipError_t launch_smla_bwd_split(const uint16_t* q, const uint16_t* kv, const uint16_t* dout, const int* idx,
                                 const float* lse, const float* delta, uint16_t* dq, uint16_t* dkv, void* workspace,
                                 int T, int Tk, int H, int K, float scale, hipStream_t stream) {
  const SplitLayout L = split_layout(T, Tk, H, K);
  char* ws = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(ws + L.part);
  int* pos = reinterpret_cast<int*>(ws + L.pos);
  int* off = reinterpret_cast<int*>(ws + L.off);
  int* hist = reinterpret_cast<int*>(ws + L.hist);
  int* sums = reinterpret_cast<int*>(ws + L.sums);
  int* kbuf[2] = {reinterpret_cast<int*>(ws + L.k0), reinterpret_cast<int*>(ws + L.k1)};
  int* vbuf[2] = {reinterpret_cast<int*>(ws + L.v0), reinterpret_cast<int*>(ws + L.v1)};
  const int* keys = nullptr;
  const int* vals = nullptr;
  int shift = 0;
  for (int ps = 0; ps < L.n_pass; ps++) {
    const int bits = ps == 0 ? L.bits0 : L.bits1;
    hipLaunchKernelGGL(sort_hist_kernel, dim3(L.n_tiles), dim3(kSortThreads), 0, stream, keys, idx, Tk, L.n, shift,
                       bits, L.n_tiles, hist);
    const hipError_t e = launch_scan(hist, ((long long)1 << bits) * L.n_tiles, sums, L.n_scan_blocks, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sort_scatter_kernel, dim3(L.n_tiles), dim3(kSortThreads), 0, stream, keys, vals, idx, Tk, L.n,
                       shift, bits, L.n_tiles, hist, kbuf[ps], vbuf[ps], ps == L.n_pass - 1 ? pos : nullptr);
    keys = kbuf[ps];
    vals = vbuf[ps];
    shift += bits;
  }
  hipLaunchKernelGGL(row_offsets_kernel, dim3((unsigned)((Tk + 256) / 256)), dim3(256), 0, stream, keys, L.n, Tk, off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_smla_bwd_partial(q, kv, dout, idx, lse, delta, dq, part, pos, T, Tk, H, K, scale, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dkv_sum_kernel, dim3(Tk), dim3(kSumGroups * kSumCols), 0, stream, part, off, L.n, L.n_ht, dkv);
  return hipGetLastError();
}

}  // namespace mi355
