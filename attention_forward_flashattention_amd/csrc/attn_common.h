// attn_common.h — device helpers shared by the forward and backward kernels
// (gfx950: wave64, 32x32x16 bf16 MFMA, direct global-to-LDS loads, LDS
// transpose reads).  Private to the library sources.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace attn_detail {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float floatx16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int uint4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int uint2_t;
typedef __attribute__((ext_vector_type(2))) float floatx2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int kListBlock = 128;  // block-list / block-mask granularity (rows and keys)
// KV iteration modes: every key, an ordered block list, a bit-packed block
// mask, an ordered block list walked with ordered skipping
enum { kDense = 0, kList = 1, kMask = 2, kOsk = 3 };
constexpr float kLn2 = 0.69314718055994530942f;
// s_waitcnt immediate that waits for vmcnt == 0 and leaves the other counters
// free (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14])
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);
// ... and the immediate that waits for vmcnt <= n (n < 64)
constexpr int wait_vmcnt(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }


// ---------------------------------------------------------------------------
// LDS layouts (rows of D bf16 values; bank behaviour measured with the
// SQ_LDS_BANK_CONFLICT counter on gfx950).
//  K and Q: 16 B chunks XOR-swizzled by row, so the 16 consecutive rows that
//    one MFMA operand read touches at one logical chunk hit 16 distinct
//    4-bank groups (ds_read_b128, conflict-free).
//  V: 64 B pairs of 32 B units XOR-swizzled by row, so the 4 rows x 64 B that
//    32 lanes of one transpose read touch land in 4 distinct 64 B bank ranges
//    (ds_read_b64_tr_b16, conflict-free).
// ---------------------------------------------------------------------------
template <int D>
struct Lds {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                       // 16 B chunks per row
  static constexpr int kRowsPerWin = kRowBytes >= 256 ? 1 : 256 / kRowBytes;
  static constexpr int kPairs = D / 32;                       // 64 B pairs per row
  static constexpr int kPairSwz = kPairs < 4 ? kPairs : 4;
  __device__ static __forceinline__ int kswz(int r) { return (r / kRowsPerWin) % kChunks; }
  // byte offset of 16 B chunk `c` of row `r` (K / Q layout)
  __device__ static __forceinline__ int kq(int r, int c) {
    return r * kRowBytes + ((c ^ kswz(r)) << 4);
  }
  __device__ static __forceinline__ int vswz(int r) { return (r / kRowsPerWin) % kPairSwz; }
  // byte offset of byte `b` (0..31) of 32 B unit `u` of row `r` (V layout)
  __device__ static __forceinline__ int vv(int r, int u, int b) {
    return r * kRowBytes + ((((u >> 1) ^ vswz(r)) << 6) | ((u & 1) << 5)) + b;
  }
  // logical 16 B chunk that the V layout stores in physical chunk `pc` of row `r`
  __device__ static __forceinline__ int v_logical_chunk(int r, int pc) {
    return ((((pc >> 2) ^ vswz(r))) << 2) | (pc & 3);
  }
};

// Dual layout, for tiles that are read both row-wise (ds_read_b128, one row
// per lane) and column-wise (ds_read_b64_tr_b16).  16 B chunk c of row r sits
// at physical chunk c ^ f(r).  f takes 16 distinct values over any 16
// consecutive rows, so a row-wise read of 16 rows at one chunk hits 16
// distinct 16 B bank slots; and over 4 aligned consecutive rows f differs in
// the bits that pick a 64 B bank range within a 256 B bank window, so the
// 4 rows x 64 B of one transpose read land in 4 distinct ranges.  (At
// head_dim 64 two rows share a window: f then uses bit 1 of r in place of
// bit 0.)
template <int D>
struct Dual {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;
  __host__ __device__ static constexpr int f(int r) {
    return D == 64 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) : (((r & 3) << 2) | ((r >> 2) & 3));
  }
  // byte offset of 16 B chunk `c` of row `r`; f is periodic in r with period
  // 16, so row offsets that are multiples of 16 can be added as immediates
  __host__ __device__ static constexpr int at(int r, int c) {
    return r * kRowBytes + ((c ^ f(r)) << 4);
  }
};

// Compile-time LDS buffer index of a main-loop step.
template <int B>
struct BufTag {
  static constexpr int value = B;
};

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, so that i can be
// used as a template argument (immediate offsets of inline assembly).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Byte offset (within a V tile) of the rows read by PV step i: dt = i % kDt,
// (kt, c) = i / kDt; a step reads 16 keys starting at key 32 kt + 16 c.
template <class L, int kDt>
__host__ __device__ constexpr int tr_off(int i) {
  return ((i / kDt) >> 1) * 32 * L::kRowBytes + ((i / kDt) & 1) * 16 * L::kRowBytes;
}

// Two LDS transpose reads (rows +0 and +kRow8 bytes apart: keys +0..7 and
// +8..15 of a 16-key group) forming one MFMA A operand.  Written as inline
// assembly: the compiler builtin for this read makes the compiler wait for every direct
// global-to-LDS load in flight before it (the prefetch of the next tile),
// which the double-buffered layout never needs.  The caller waits for the
// result with lgkm_wait before using it.
template <int kOff, int kRow8>
__device__ __forceinline__ bf16x8_t tr_pair(uint32_t addr) {
  uint2_t lo, hi;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(addr), "i"(kOff));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(addr), "i"(kOff + kRow8));
  const uint4_t packed = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8_t, packed);
}

// Two LDS transpose reads from separate per-lane addresses (immediate offset
// kOff on both), forming one MFMA operand: lo from `a`, hi from `b`.
template <int kOff>
__device__ __forceinline__ bf16x8_t tr_pair2(uint32_t a, uint32_t b) {
  uint2_t lo, hi;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(a), "i"(kOff));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(b), "i"(kOff));
  const uint4_t packed = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8_t, packed);
}

// One 16 B LDS read (an MFMA operand) at a per-lane address plus an immediate
// offset.  Inline assembly for the same reason as tr_pair; the caller waits
// for the result with lgkm_wait.
template <int kOff>
__device__ __forceinline__ bf16x8_t ld_b128(uint32_t addr) {
  uint4_t x;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(x) : "v"(addr), "i"(kOff));
  return __builtin_bit_cast(bf16x8_t, x);
}

// Wait until at most N LDS operations are outstanding; `x` is tied through so
// its uses cannot move above the wait.
template <int N>
__device__ __forceinline__ void lgkm_wait(bf16x8_t &x) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}

// Sum of x over the 64 lanes of a wave (every lane gets the sum).
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ uint4_t ld_global16(const uint16_t *p) {
  return *reinterpret_cast<const uint4_t *>(p);
}

// Exchange between the two lane halves: after v_permlane32_swap, `a` holds
// lanes 0-31 of x in both halves and `b` lanes 32-63 of x in both halves, so
// a (op) b is the pairwise result for lanes l and l^32 in every lane.  (Inline
// assembly: the compiler builtin returns the same register for both results.)
__device__ __forceinline__ void half_pair(float x, float &a, float &b) {
  a = x;
  b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float half_max(float x) {
  float a, b;
  half_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float half_sum(float x) {
  float a, b;
  half_pair(x, a, b);
  return a + b;
}

}  // namespace attn_detail
