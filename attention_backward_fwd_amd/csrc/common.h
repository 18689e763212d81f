// Device helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D = A(16x32) * B(32x16) + C, bf16 in, fp32 accumulate.  Lane l (r = l % 16,
// g = l / 16) supplies A[r][8g .. 8g+7] and B[8g .. 8g+7][r]; result element j
// of lane l is C[4g + j][r].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A(32x16) * B(16x32) + C on the matrix cores, bf16 in, fp32 accumulate.
// Lane l (r = l % 32, g = l / 32) supplies A[r][8g .. 8g+7] and B[8g .. 8g+7][r];
// result element j of lane l is C[8*(j/4) + 4*g + j%4][r].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of element j of a 32x32 result held by a lane of half hi (= l / 32).
__device__ __forceinline__ int c_row(int j, int hi) { return 8 * (j >> 2) + 4 * hi + (j & 3); }

// LDS transposing read of four 16-bit values.  Within each group of 16 lanes,
// element e of lane i comes from the 8-byte chunk addressed by lane 4*e + i/4,
// at position i % 4.  Four lanes pointing at consecutive 4-element chunks of
// one row therefore hand out that row's 16 values one per lane.
__device__ __forceinline__ i16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// Two transposing reads forming one 8-value MFMA operand.
__device__ __forceinline__ bf16x8 lds_read_tr8(const uint16_t* p0, const uint16_t* p1) {
  i16x4 a = lds_read_tr(p0);
  i16x4 b = lds_read_tr(p1);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// The same reads at a byte offset from an LDS array.  The array's address is
// a constant, which the compiler folds into the instruction's 16-bit offset
// field when it fits, so that reads of different arrays at the same offset
// share one address register.
__device__ __forceinline__ bf16x8 lds_b128_at(const void* base, uint32_t boff) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(base) + boff);
}
__device__ __forceinline__ bf16x8 lds_tr8_at(const void* base, uint32_t b0, uint32_t b1) {
  const char* c = reinterpret_cast<const char*>(base);
  return lds_read_tr8(reinterpret_cast<const uint16_t*>(c + b0), reinterpret_cast<const uint16_t*>(c + b1));
}

// Combine a per-lane value with the one held 32 lanes away (the other half of
// the wavefront).  permlane32_swap(x, x) returns {own, other} in the lower half
// and {other, own} in the upper half, so any symmetric operation of the pair
// is the cross-half result in every lane.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float from_bf16(uint16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                        float a6, float a7) {
  u32x4 u = {pack_bf16x2(a0, a1), pack_bf16x2(a2, a3), pack_bf16x2(a4, a5), pack_bf16x2(a6, a7)};
  return __builtin_bit_cast(bf16x8, u);
}

// ---------------------------------------------------------------- LDS tiles
// A tile holds R rows of D bf16 values, unpadded (so that the LDS-DMA loads,
// which place lane i's 16 bytes at base + 16*i, can fill it), with the
// 16-byte slot index of row r XORed by swz<D>(r).  The swizzle is chosen so
// that both access patterns of the kernels are free of bank conflicts:
//   * 16-byte row reads (MFMA A operands): 16 consecutive rows, same slot;
//   * transposing 8-byte reads: 4 consecutive rows (first one a multiple of
//     4) x 4 consecutive slots.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);  // 16 slots per 256-byte row
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);              // 8 slots per 128-byte row
}

// Element offset of (row, col) in a swizzled tile; col is a multiple of 4.
template <int D>
__device__ __forceinline__ int swz_off(int row, int col) {
  return row * D + ((((col >> 3) ^ swz<D>(row))) << 3) + (col & 7);
}

// Because the swizzle is an XOR on the slot index, moving the column by a
// multiple of 8 elements whose bits do not overlap the starting slot turns
// into an XOR of the element offset: swz_off(r, c + 8k) == swz_off(r, c) ^ 8k
// when (c >> 3) & k == 0.  Row moves by multiples of 16 keep swz() unchanged
// and are plain additions.  The kernels build one offset per lane and derive
// the rest this way.
__device__ __forceinline__ int xslot(int off, int k8) { return off ^ k8; }

// Keep the compiler from hoisting values derived from v out of a loop: v
// becomes opaque at this point (scalar / per-lane variants).
template <typename T>
__device__ __forceinline__ T opaque(T v) {
  asm volatile("" : "+s"(v));
  return v;
}
template <typename T>
__device__ __forceinline__ T opaque_v(T v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(void* p) {
  return (__attribute__((address_space(3))) void*)(p);
}

// Asynchronous global -> LDS copy of rows [row0, row0 + R) of a row-major
// bf16 matrix with row stride rs elements into a swizzled tile.  Rows at or
// past `nrows` read row nrows - 1 instead (callers mask them); every source
// address is therefore inside the matrix.  Each wave instruction moves 1 KB;
// the NW waves of the workgroup split the tile (waves w >= R*D/512 issue
// nothing when the tile is smaller than NW KB).  Completion: vmcnt.
template <int D, int R, int NW = 4>
__device__ __forceinline__ void tile_load_async(const uint16_t* g, size_t rs, int row0, int nrows,
                                                uint16_t* tile, int w, int lane) {
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;    // rows per wave instruction
  constexpr int NI = R / RPI;      // wave instructions per tile
  static_assert(NI % NW == 0 || NI < NW, "tile must split evenly over the waves");
  const int rl = lane / CPR, slot = lane % CPR;
  const uint16_t* base = g + (size_t)row0 * rs;  // wave-uniform
  const int last = nrows - 1 - row0;
#pragma unroll
  for (int j = w; j < NI; j += NW) {
    const int r = j * RPI + rl;
    // 32-bit per-lane byte offset from the uniform row base.
    const uint32_t off = ((uint32_t)min(r, last) * (uint32_t)rs + (uint32_t)((slot ^ swz<D>(r)) << 3)) * 2u;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(base) + off, lds_ptr(tile + j * 512), 16, 0, 0);
  }
}

// Workgroup barrier for LDS hand-offs only.  Waves of these kernels exchange
// data through LDS alone, so a wave only has to finish its own LDS
// instructions (lgkmcnt) before the barrier; in particular it does not wait
// for its outstanding global loads, LDS-DMA loads, stores or atomics (an
// LDS-scoped fence would, because LDS-DMA writes count as LDS writes).  The
// LDS-DMA loads are waited for explicitly (wait_vmem / wait_vmem_but) where
// their data is needed.  The "memory" clobber keeps the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 8-byte LDS store issued as inline assembly.  The compiler's LDS-DMA
// tracking does not see it, so it is not held back behind LDS-DMA loads in
// flight to other buffers.  Ordering with lds_barrier() (also volatile asm)
// is preserved; the compiler's own lgkmcnt waits only become stricter.
__device__ __forceinline__ void lds_store_b64_asm(uint16_t* p, u32x2 v) {
  const uint32_t addr = (uint32_t)(uintptr_t)lds_ptr(p);
  asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(v));
}
// Same, at an LDS byte address.
__device__ __forceinline__ void lds_store_b64_addr(uint32_t addr, u32x2 v) {
  asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(v));
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)lds_ptr(const_cast<void*>(p));
}
// LDS-DMA loads issued as inline assembly (16 or 4 bytes per lane, from a
// per-lane global address to `lds` + 16 (or 4) * lane; `lds` wave-uniform,
// placed in M0 by the compiler).  The compiler does not know that they write
// LDS, so it adds no waits of its own for them: the caller waits
// (wait_vmem / wait_vmem_but) and synchronises (lds_barrier) before any LDS
// read of the data.  The s_nop separates the M0 write from the load.
__device__ __forceinline__ void dma_b128_asm(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
// The same from g + OFF bytes.  The instruction's immediate offset moves
// the LDS destination as well as the global address, so M0 takes lds - OFF
// (lds >= OFF).
template <int OFF>
__device__ __forceinline__ void dma_b128_asm_off(const void* g, uint32_t lds) {
  static_assert(OFF >= 0 && OFF < 4096, "immediate offset");
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2" ::"v"(g), "{m0}"(lds - OFF), "i"(OFF)
               : "memory");
}
__device__ __forceinline__ void dma_b32_asm(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
// The same copy issued as inline assembly (dma_b128_asm): the compiler adds
// no waits for it; the caller waits explicitly.  NI / NW instructions per
// wave (all waves when the tile is at least NW KB).
// LDS-DMA instructions tile_load_async_asm<D, R, NW> issues per wave.
template <int D, int R, int NW>
constexpr int tile_load_ops() {
  return R / (64 / (D / 8)) / NW;
}
template <int D, int R, int NW = 4>
__device__ __forceinline__ void tile_load_async_asm(const uint16_t* g, size_t rs, int row0, int nrows,
                                                    uint16_t* tile, int w, int lane) {
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;
  constexpr int NI = R / RPI;
  static_assert(NI % NW == 0, "tile must split evenly over the waves");
  const int rl = lane / CPR, slot = lane % CPR;
  const char* base = reinterpret_cast<const char*>(g + (size_t)row0 * rs);
  const int last = nrows - 1 - row0;
#pragma unroll
  for (int j = w; j < NI; j += NW) {
    const int r = j * RPI + rl;
    const uint32_t off = ((uint32_t)min(r, last) * (uint32_t)rs + (uint32_t)((slot ^ swz<D>(r)) << 3)) * 2u;
    dma_b128_asm(base + off, lds_addr(tile + j * 512));
  }
}

// 16-byte LDS store and load the compiler does not track either (see
// lds_store_b64_asm).  A load's result is only ready after lds_wait4().
__device__ __forceinline__ void lds_store_b128_addr(uint32_t addr, f32x4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v));
}
__device__ __forceinline__ f32x4 lds_load_b128_addr(uint32_t addr) {
  f32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
// Wait for this wave's LDS accesses; the four registers pass through the
// wait, so that nothing reads them before it.
__device__ __forceinline__ void lds_wait4(f32x4& a, f32x4& b, f32x4& c, f32x4& d) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// Asynchronous global -> LDS copy of n <= 64 consecutive fp32 values (one per
// lane, lanes >= n read the last one again) to lds[0 .. 63].
__device__ __forceinline__ void row_load_async(const float* g, int n, float* lds, int lane) {
  __builtin_amdgcn_global_load_lds(g + min(lane, n - 1), lds_ptr(lds), 4, 0, 0);
}

// Wait until every vector-memory operation of this wave (including LDS-DMA
// writes) has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N vector-memory operations of this wave are still in
// flight.  The counter retires operations in issue order, so this waits for
// everything except the N most recent ones (e.g. fire-and-forget atomics
// issued after the loads that must be complete).
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Buffer resource for a wave-uniform base address.  The address goes
// through readfirstlane so that the descriptor is known to be uniform and
// lives in scalar registers (a descriptor the compiler believes divergent
// turns every buffer instruction into a loop over distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Workgroups are handed to the 8 XCDs round-robin (id % 8).  This maps the
// hardware id to a logical id so that consecutive logical ids run on the same
// XCD and share its L2.  Identity when the grid is not a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  constexpr int X = 8;
  if (nwg % X) return bid;
  return (bid % X) * (nwg / X) + bid / X;
}

}  // namespace mi355
