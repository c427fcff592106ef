// attn_bwd.hip — softmax-attention backward for AMD Instinct MI355X (gfx950).
//
// Two kernels, launched in this order on the caller's stream:
//
//  1. dQ kernel: one workgroup per 128-row query tile of one (sequence, query
//     head), four wave64s of 32 rows each, like the forward.  It first forms
//     each row's D = dO.O and base-2 LSE and stores them to the workspace.
//     Then, for every KV tile of 64 keys it may see (double-buffered in LDS
//     by direct global-to-LDS loads), it recomputes the transposed tiles
//     S^T = K Q^T and dP^T = V dO^T with 32x32x16 bf16 MFMAs (lane = query
//     row, as in the forward), forms dS^T = P^T (dP^T - D) in registers and
//     accumulates dQ^T += K^T dS^T, with K^T operands read by LDS transpose
//     reads and dS^T staying in registers.
//
//  2. dK/dV kernel: one workgroup per 128-key block of one (sequence, KV
//     head), four wave64s of 32 keys each, the K and V rows of its keys in
//     registers for the whole kernel.  For every query head of the group and
//     every 64-row query tile that may see its keys, it streams Q, dO and the
//     two per-row workspace values into LDS and computes S = Q K^T and
//     dP = dO V^T with lane = key.  P and dS then leave the MFMA already in
//     the layout of the A operand of dV += P^T dO and dK += dS^T Q, whose dO
//     and Q operands come from LDS transpose reads.
//
// The gradients are the chain rule of the forward (softmax Jacobian
// dS = P (dP - D), with P recomputed from the saved LSE).  With a block
// mask, both kernels visit only the 128 x 128 blocks whose bit is set, the
// sparse backward navigation of the AdaSplash-2 explainer (section 2).
// Neither kernel uses atomics: every output element is written once, by the
// workgroup that owns it, so results are deterministic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "attn_bwd.h"
#include "attn_common.h"

namespace {

using namespace attn_detail;

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kMaxQBlocks = 16384;  // column bitmap capacity of the dK/dV kernel (mask mode)
constexpr int64_t kMaxRowStride = int64_t(1) << 24;  // Q / dO row strides, elements (32-bit tile offsets)

struct BwdParams {
  const uint16_t *q, *k, *v, *o, *g;  // g = dO
  const float *lse;
  uint16_t *dq, *dk, *dv;
  float *ws_lse2, *ws_d;  // workspace: base-2 LSE (+inf for rows that see nothing), D = dO.O
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t g_sb, g_ss, g_sh;
  int64_t dq_sb, dq_ss, dq_sh;
  int64_t dk_sb, dk_ss, dk_sh;
  int64_t dv_sb, dv_ss, dv_sh;
  const int32_t *cu;
  const uint32_t *mask;
  int64_t mask_ss, mask_sh;
  int mask_words;
  int batch, seqlen, hq, hkv, group;
  int n_tiles;    // tiles of 128 per unit (query tiles for dQ, key blocks for dK/dV)
  int n_units;    // (sequence, head) units: batch*hq for dQ, batch*hkv for dK/dV
  int unit_group; // consecutive units kept on one XCD (the query heads of one KV head for dQ)
  int xcd_remap;  // 1 when n_units % (8 * unit_group) == 0
  float c;        // scale * log2(e)
  float scale;
};

// Workgroup id -> (tile, unit), dealing workgroups round-robin over the 8 XCDs
// with the units of one group on one XCD (as the forward does); `reverse`
// issues the last tiles first (the heaviest ones for causal dQ).
__device__ __forceinline__ void decode(const BwdParams &p, bool reverse, int &tile, int &unit) {
  const int w = blockIdx.x;
  int rank;
  if (p.xcd_remap) {
    const int upx = p.n_units >> 3;
    const int xcd = w & 7;
    const int local = w >> 3;
    rank = local / upx;
    const int lu = local % upx;
    unit = ((lu / p.unit_group) * 8 + xcd) * p.unit_group + lu % p.unit_group;
  } else {
    rank = w / p.n_units;
    unit = w % p.n_units;
  }
  tile = reverse ? p.n_tiles - 1 - rank : rank;
}

// Index of (sequence b, query head h, row) in the caller's lse array.
__device__ __forceinline__ int64_t lse_index(const BwdParams &p, int b, int h, int64_t tok0,
                                             int64_t total, int row) {
  if (p.cu) return (int64_t)h * total + tok0 + row;
  return ((int64_t)b * p.hq + h) * p.seqlen + row;
}

// Index of (sequence b, query head h, row) in the workspace arrays: one slot of
// seqlen rows per (sequence, head), packed or not, so every row below seqlen
// stays inside the workspace.
__device__ __forceinline__ int64_t ws_index(const BwdParams &p, int b, int h, int row) {
  return ((int64_t)b * p.hq + h) * p.seqlen + row;
}

__device__ __forceinline__ float dot8(uint4_t a, uint4_t b) {
  const bf16x8_t x = __builtin_bit_cast(bf16x8_t, a);
  const bf16x8_t y = __builtin_bit_cast(bf16x8_t, b);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = __builtin_fmaf((float)x[e], (float)y[e], s);
  return s;
}

// Direct global -> LDS loads of two tiles of rows (each wave-wide load fills
// 64 consecutive 16 B LDS slots; lane load n fetches the 16 B at byte offset
// aoff[n] / boff[n] from the tiles' first rows a / b, row lrow0 + n * kRowStep
// of the tile).  The offsets are 32-bit (the row strides accepted keep a
// tile's rows within 4 GB of its first) and stay so at the load (the empty
// asm), so each load takes one register offset from a scalar base.  Rows at
// or beyond rows_left re-read row rows_left - 1; a tile that starts at or
// past the end (rows_left <= 0) moves its base back to that row, so that no
// lane steps back by more than its own row.  (A device function rather than
// a lambda: the LDS pointer casts of the load builtin inside a lambda leave
// the kernel without its host stub.)
template <int kLoads, int kRowStep>
__device__ __forceinline__ void issue_pair(char *la, char *lb, const char *a, const char *b,
                                           const uint32_t *aoff, const uint32_t *boff, int lrow0,
                                           uint32_t a_ssb, uint32_t b_ssb, int rows_left) {
  const int r_last = rows_left - 1;
  const int base_row = min(r_last, 0);
  const char *const ta = a + (int64_t)base_row * a_ssb;
  const char *const tb = b + (int64_t)base_row * b_ssb;
#pragma unroll
  for (int n = 0; n < kLoads; ++n) {
    const int lrow = lrow0 + n * kRowStep;
    const uint32_t back = (uint32_t)(max(lrow - r_last, 0) + base_row);  // 0 <= back <= lrow
    uint32_t oa = aoff[n] - back * a_ssb, ob = boff[n] - back * b_ssb;
    asm volatile("" : "+v"(oa), "+v"(ob));
    __builtin_amdgcn_global_load_lds(ta + oa, (lds_void_t *)(la + n * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(tb + ob, (lds_void_t *)(lb + n * 1024), 16, 0, 0);
  }
}

// issue_pair for a tile wholly inside the sequence (no row clamping).
template <int kLoads>
__device__ __forceinline__ void issue_pair_full(char *la, char *lb, const char *a, const char *b,
                                                const uint32_t *aoff, const uint32_t *boff) {
#pragma unroll
  for (int n = 0; n < kLoads; ++n) {
    uint32_t oa = aoff[n], ob = boff[n];
    asm volatile("" : "+v"(oa), "+v"(ob));
    __builtin_amdgcn_global_load_lds(a + oa, (lds_void_t *)(la + n * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(b + ob, (lds_void_t *)(lb + n * 1024), 16, 0, 0);
  }
}

// Load n of a whole tile's rows (as issue_pair_full does for every n), for
// callers that spread the loads over other work.
template <int kN>
__device__ __forceinline__ void issue_one(char *l, const char *g, const uint32_t *off) {
  uint32_t o = off[kN];
  asm volatile("" : "+v"(o));
  __builtin_amdgcn_global_load_lds(g + o, (lds_void_t *)(l + kN * 1024), 16, 0, 0);
}

// One dword per lane from global to 64 consecutive LDS dwords.
__device__ __forceinline__ void issue_dwords(char *l, const float *src) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t *)l, 4, 0, 0);
}

// ===========================================================================
// dQ kernel
// ===========================================================================
// Workgroups per CU of the dQ kernel: two up to head_dim 128; at 256 the Q,
// dO and dQ registers of a wave's 32 rows (~380) leave one wave per SIMD.
template <int D>
constexpr int dq_min_blocks() {
  return D == 256 ? 1 : 2;
}

template <int D, bool CAUSAL, int MODE>
__global__ __launch_bounds__(256, dq_min_blocks<D>()) void attn_bwd_dq_kernel(BwdParams p) {
  using LK = Dual<D>;  // K tile: row-wise reads (S^T) and transpose reads (dQ^T)
  using LV = Lds<D>;   // V tile: row-wise reads only
  constexpr int kNW = 4;
  constexpr int kBM = 32 * kNW;
  // keys per KV tile (32 at head_dim 256: LDS operand offsets stay below 64 KiB)
  constexpr int kBN = D == 256 ? 32 : 64;
  constexpr int kRowBytes = D * 2;
  constexpr int kChunks = D / 8;
  constexpr int kDc = D / 16;
  constexpr int kDt = D / 32;
  constexpr int kKt = kBN / 32;
  constexpr int kTileBytes = kBN * kRowBytes;
  constexpr int kBufBytes = 2 * kTileBytes;  // K tile then V tile
  constexpr int kLoads = kTileBytes / 1024 / kNW;
  static_assert(kLoads * 1024 * kNW == kTileBytes, "tile must split evenly over waves");
  __shared__ __attribute__((aligned(1024))) char smem[2 * kBufBytes];

  int tile, unit;
  decode(p, CAUSAL || MODE != kDense, tile, unit);
  const int b = unit / p.hq;
  const int h = unit % p.hq;
  const int kvh = h / p.group;
  int64_t tok0 = 0, total = 0;
  int len = p.seqlen;
  if (p.cu) {
    tok0 = p.cu[b];
    len = min(p.cu[b + 1] - p.cu[b], p.seqlen);  // seqlen bounds every length
    total = p.cu[p.batch];
  }
  const int q0 = tile * kBM;
  if (q0 >= len) return;

  const uint16_t *qg = p.q + (p.cu ? tok0 * p.q_ss : (int64_t)b * p.q_sb) + (int64_t)h * p.q_sh;
  const uint16_t *og = p.o + (p.cu ? tok0 * p.o_ss : (int64_t)b * p.o_sb) + (int64_t)h * p.o_sh;
  const uint16_t *gg = p.g + (p.cu ? tok0 * p.g_ss : (int64_t)b * p.g_sb) + (int64_t)h * p.g_sh;
  const uint16_t *kg = p.k + (p.cu ? tok0 * p.k_ss : (int64_t)b * p.k_sb) + (int64_t)kvh * p.k_sh;
  const uint16_t *vg = p.v + (p.cu ? tok0 * p.v_ss : (int64_t)b * p.v_sb) + (int64_t)kvh * p.v_sh;
  uint16_t *dqg = p.dq + (p.cu ? tok0 * p.dq_ss : (int64_t)b * p.dq_sb) + (int64_t)h * p.dq_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int j16 = lane & 15;

  // ---- KV iteration space: every KV tile of 64 keys up to the causal limit,
  // or the two tiles of every 128-key block whose mask bit is set
  constexpr int kSub = kListBlock / kBN;
  const int n_kvblk = (len + kListBlock - 1) / kListBlock;
  const uint32_t *mrow = nullptr;
  const int m_lim = CAUSAL ? min(n_kvblk, tile + 1) : n_kvblk;
  const int m_words = (m_lim + 31) >> 5;
  auto m_valid = [&](int w) -> uint32_t {
    const int left = m_lim - 32 * w;
    return left >= 32 ? 0xffffffffu : (left <= 0 ? 0u : ((1u << left) - 1u));
  };
  int n_iter;
  if (MODE == kMask) {
    mrow = p.mask + b * p.mask_ss + kvh * p.mask_sh + (int64_t)tile * p.mask_words;
    int n_blk = 0;
    for (int w = 0; w < m_words; ++w) n_blk += __builtin_popcount(mrow[w] & m_valid(w));
    n_iter = n_blk * kSub;
  } else {
    const int kv_end = CAUSAL ? min(len, q0 + kBM) : len;
    n_iter = (kv_end + kBN - 1) / kBN;
  }
  int m_w = -1;
  uint32_t m_bits = 0;
  int m_blk = 0;
  auto kv_start = [&](int it) -> int {  // called for it = 0, 1, 2, ... in order
    if (MODE == kDense) return it * kBN;
    if (it % kSub == 0) {
      while (m_bits == 0) {
        if (++m_w >= m_words) return -1;
        m_bits = mrow[m_w] & m_valid(m_w);
      }
      m_blk = 32 * m_w + __builtin_ctz(m_bits);
      m_bits &= m_bits - 1u;
    }
    return m_blk * kListBlock + (it % kSub) * kBN;
  };

  // ---- direct global -> LDS loads of one KV tile (K in the dual layout, V in
  // the row-read layout); rows past the end of the sequence re-read the last
  // row (finite data; those keys are masked)
  // (byte offsets of this lane's loads within a tile's rows; row of load n:
  // lrow0 + n * kRowStep)
  constexpr int kRowStep = 64 / kChunks;
  static_assert(64 % kChunks == 0, "a wave-wide load covers whole rows");
  uint32_t koff[kLoads], voff[kLoads];
  const int slot_byte0 = wave * kLoads * 1024;
  const int lrow0 = (wave * kLoads * 64 + lane) / kChunks;
  const uint32_t k_ssb = (uint32_t)p.k_ss * 2u, v_ssb = (uint32_t)p.v_ss * 2u;  // row strides in bytes
#pragma unroll
  for (int n = 0; n < kLoads; ++n) {
    const int slot = (wave * kLoads + n) * 64 + lane;
    const int r = slot / kChunks, pc = slot % kChunks;
    koff[n] = (uint32_t)r * k_ssb + (uint32_t)(pc ^ LK::f(r)) * 16u;
    voff[n] = (uint32_t)r * v_ssb + (uint32_t)(pc ^ LV::kswz(r)) * 16u;
  }
  const char *const kgb = reinterpret_cast<const char *>(kg);
  const char *const vgb = reinterpret_cast<const char *>(vg);
  auto issue = [&](int buf, int kv) {
    char *kb = smem + buf * kBufBytes + slot_byte0;
    const char *const kt = kgb + (int64_t)kv * k_ssb;
    const char *const vt = vgb + (int64_t)kv * v_ssb;
    if (len - kv >= kBN)
      issue_pair_full<kLoads>(kb, kb + kTileBytes, kt, vt, koff, voff);
    else
      issue_pair<kLoads, kRowStep>(kb, kb + kTileBytes, kt, vt, koff, voff, lrow0, k_ssb, v_ssb, len - kv);
  };

  int kv_cur = n_iter > 0 ? kv_start(0) : -1;
  if (kv_cur >= 0) issue(0, kv_cur);

  // ---- this lane's query row: Q and dO as MFMA B operands (head-dim values
  // 16 dc + 8 hi .. +7), D = dO.O and the base-2 LSE; rows past the end read
  // as zero and get P = 0 (LSE +inf)
  const int qrow = q0 + wave * 32 + l32;
  const int wq_last = q0 + wave * 32 + 31;
  bf16x8_t qreg[kDc], greg[kDc];
  float dpart = 0.f;
#pragma unroll
  for (int dc = 0; dc < kDc; ++dc) {
    uint4_t x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u}, z = {0u, 0u, 0u, 0u};
    if (qrow < len) {
      x = ld_global16(qg + (int64_t)qrow * p.q_ss + dc * 16 + hi * 8);
      y = ld_global16(gg + (int64_t)qrow * p.g_ss + dc * 16 + hi * 8);
      z = ld_global16(og + (int64_t)qrow * p.o_ss + dc * 16 + hi * 8);
    }
    qreg[dc] = __builtin_bit_cast(bf16x8_t, x);
    greg[dc] = __builtin_bit_cast(bf16x8_t, y);
    dpart += dot8(y, z);
  }
  const float drow = half_sum(dpart);
  float lse2 = INFINITY;
  if (qrow < len) {
    const float l = p.lse[lse_index(p, b, h, tok0, total, qrow)];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    if (hi == 0) {
      const int64_t w = ws_index(p, b, h, qrow);
      p.ws_lse2[w] = lse2;
      p.ws_d[w] = drow;
    }
  }

  floatx16_t acc[kDt];
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  // per-lane LDS offsets: row-wise reads of K and V (row l32, chunk 2 dc + hi)
  // and the two transpose reads of K^T (rows 4 hi + j16/4 and 8 more, the
  // 4 columns at 32 dt + 16 (l32/16) + 4 (j16%4))
  uint32_t kaddr[kDc], vaddr[kDc];
  uint32_t ta[kDt], tb[kDt];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_char_t *)smem;
#pragma unroll
  for (int dc = 0; dc < kDc; ++dc) {
    kaddr[dc] = smem_lds + LK::at(l32, 2 * dc + hi);
    vaddr[dc] = smem_lds + kTileBytes + LV::kq(l32, 2 * dc + hi);
    asm volatile("" : "+v"(kaddr[dc]));
    asm volatile("" : "+v"(vaddr[dc]));
  }
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt) {
    const int ch = 4 * dt + 2 * (l32 >> 4) + ((j16 & 3) >> 1);
    ta[dt] = smem_lds + LK::at(4 * hi + (j16 >> 2), ch) + (j16 & 1) * 8;
    tb[dt] = smem_lds + LK::at(8 + 4 * hi + (j16 >> 2), ch) + (j16 & 1) * 8;
    asm volatile("" : "+v"(ta[dt]));
    asm volatile("" : "+v"(tb[dt]));
  }

  auto step = [&](const int it, auto buf_tag) {
    constexpr int kBuf = decltype(buf_tag)::value;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    int kv_nxt = -1;
    if (it + 1 < n_iter) {
      kv_nxt = kv_start(it + 1);
      if (kv_nxt >= 0) issue(1 - kBuf, kv_nxt);
    }
    const int kv0 = kv_cur;
    kv_cur = kv_nxt;
    if (kv0 < 0) return;
    if (CAUSAL && kv0 > wq_last) return;
    const bool need_mask = (kv0 + kBN > len) || (CAUSAL && kv0 + kBN - 1 > q0 + wave * 32);
    // key kv0 + 32 kt + hi*4 + o (o a compile-time offset) is masked when o > lim - 32 kt
    const int lim = (CAUSAL ? min(qrow, len - 1) : len - 1) - kv0 - hi * 4;
    // one 32-key half of the tile at a time (bounds the live registers)
    static_for<kKt>([&](auto KT) {
      constexpr int kt = decltype(KT)::value;
      if (CAUSAL && kv0 + kt * 32 > wq_last) return;  // this half lies above every row
      // ---- S^T = K Q^T and dP^T = V dO^T (32 keys x 32 query rows)
      // (operand reads four MFMAs ahead, each waited for exactly: LDS reads
      // complete in order; step i: S (even i, a K row) or dP (odd i, a V
      // row) of head-dim chunk i / 2)
      floatx16_t s, dp;
      {
        constexpr int kRing = 4;
        constexpr int kSteps = 2 * kDc;
        constexpr int kOff = kBuf * kBufBytes + kt * 32 * kRowBytes;
        auto load = [&](auto T) __attribute__((always_inline)) -> bf16x8_t {
          constexpr int t = decltype(T)::value;
          if constexpr (t & 1)
            return ld_b128<kOff>(vaddr[t >> 1]);
          else
            return ld_b128<kOff>(kaddr[t >> 1]);
        };
        bf16x8_t ring[kRing];
        static_for<kRing>([&](auto T) { ring[decltype(T)::value] = load(T); });
        static_for<kSteps>([&](auto I) {
          constexpr int i = decltype(I)::value;
          constexpr int dc = i >> 1;
          lgkm_wait<(kSteps - 1 - i < kRing - 1 ? kSteps - 1 - i : kRing - 1)>(ring[i % kRing]);
          if constexpr (i & 1) {
            if constexpr (dc == 0)
              dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], greg[dc], floatx16_t{}, 0, 0, 0);
            else
              dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], greg[dc], dp, 0, 0, 0);
          } else {
            if constexpr (dc == 0)
              s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], qreg[dc], floatx16_t{}, 0, 0, 0);
            else
              s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], qreg[dc], s, 0, 0, 0);
          }
          if constexpr (i + kRing < kSteps) ring[i % kRing] = load(std::integral_constant<int, i + kRing>{});
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      // ---- P^T = 2^(c s - lse2) with the causal diagonal and sequence tail
      // masked, dS^T = P^T (dP^T - D), rounded to bf16 in the B operand
      // layout (MFMA k index e of step c = key 32 kt + 16 c + 8 (e/4) +
      // 4 hi + e%4)
      // (two copies behind a uniform branch: left to itself the compiler
      // evaluates the mask on every tile and selects)
      bf16x8_t dsb[2];
      auto ds_tile = [&](auto M) __attribute__((always_inline)) {
        constexpr bool kMask = decltype(M)::value;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.c, -lse2));
          if (kMask && kt * 32 + (i >> 2) * 8 + (i & 3) > lim) pv = 0.f;
          dsb[i >> 3][i & 7] = (__bf16)(pv * (dp[i] - drow));
        }
      };
      if (need_mask) {
        asm volatile("; masked tile");
        ds_tile(std::true_type{});
      } else {
        asm volatile("; unmasked tile");
        ds_tile(std::false_type{});
      }
      // ---- dQ^T += K^T dS^T (K^T by transpose reads four MFMAs ahead,
      // waited for exactly; consecutive MFMAs on different accumulators)
      {
        constexpr int kRing = 4;
        constexpr int kSteps = kDt * 2;  // step i: dt = i % kDt, c = i / kDt
        auto load = [&](auto T) __attribute__((always_inline)) -> bf16x8_t {
          constexpr int t = decltype(T)::value;
          return tr_pair2<kBuf * kBufBytes + (32 * kt + 16 * (t / kDt)) * kRowBytes>(ta[t % kDt], tb[t % kDt]);
        };
        bf16x8_t ring[kRing];
        static_for<kRing>([&](auto T) { ring[decltype(T)::value] = load(T); });
        static_for<kSteps>([&](auto I) {
          constexpr int i = decltype(I)::value;
          constexpr int dt = i % kDt, c = i / kDt;
          lgkm_wait<2 * (kSteps - 1 - i < kRing - 1 ? kSteps - 1 - i : kRing - 1)>(ring[i % kRing]);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], dsb[c], acc[dt], 0, 0, 0);
          if constexpr (i + kRing < kSteps) ring[i % kRing] = load(std::integral_constant<int, i + kRing>{});
          __builtin_amdgcn_sched_barrier(0);
        });
      }
    });
  };
  for (int it = 0; it < n_iter; it += 2) {
    step(it, BufTag<0>{});
    if (it + 1 < n_iter) step(it + 1, BufTag<1>{});
  }

  // ---- epilogue: dQ = scale * acc in bf16, written through LDS so that 16
  // consecutive lanes store one whole row with 16-byte stores
  __syncthreads();
  {
    constexpr int kRowsPerStore = 1024 / kRowBytes;
    char *so = smem + wave * 32 * kRowBytes;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const floatx2_t f01 = {acc[dt][g4 * 4 + 0] * p.scale, acc[dt][g4 * 4 + 1] * p.scale};
        const floatx2_t f23 = {acc[dt][g4 * 4 + 2] * p.scale, acc[dt][g4 * 4 + 3] * p.scale};
        uint2_t w;
        w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f01, bf16x2_t));
        w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(f23, bf16x2_t));
        const int ch = (dt * 4 + g4) ^ (l32 % kChunks);
        *reinterpret_cast<uint2_t *>(so + l32 * kRowBytes + ch * 16 + hi * 8) = w;
      }
    constexpr int kStores = 32 / kRowsPerStore;
    const int r0 = lane / kChunks;
    const int ch = lane % kChunks;
    uint16_t *orow = dqg + (int64_t)(q0 + wave * 32 + r0) * p.dq_ss + ch * 8;
    const int64_t step_rows = (int64_t)kRowsPerStore * p.dq_ss;
#pragma unroll
    for (int k = 0; k < kStores; ++k) {
      const int r = k * kRowsPerStore + r0;
      const uint4_t x = *reinterpret_cast<const uint4_t *>(so + r * kRowBytes + ((ch ^ (r % kChunks)) * 16));
      if (q0 + wave * 32 + r < len) *reinterpret_cast<uint4_t *>(orow + k * step_rows) = x;
    }
  }
}

// ===========================================================================
// dK/dV kernel
// ===========================================================================
// Workgroups per CU: at head_dim 128 the K/V operands and the dK/dV
// accumulators of a wave's 32 keys take ~380 registers, so one wave per SIMD;
// at head_dim 64 half that, and two workgroups share a CU.
template <int D>
constexpr int dkdv_min_blocks() {
  return D == 64 ? 2 : 1;
}
// dK/dV columns per workgroup: all of them up to head_dim 128; at 256 the K
// and V operands (the whole head dimension, for S and dP) and the
// accumulators of all 256 columns would not fit one wave's registers, so each
// workgroup takes one 128-column half of dK and dV (S and dP are formed once
// per half).
template <int D>
constexpr int dkdv_cols() {
  return D == 256 ? 128 : D;
}

template <int D, bool CAUSAL, int MODE>
__global__ __launch_bounds__(256, dkdv_min_blocks<D>()) void attn_bwd_dkdv_kernel(BwdParams p) {
  using L = Dual<D>;  // Q and dO tiles: row-wise and transpose reads
  constexpr int kNW = 4;
  constexpr int kBK = 32 * kNW;  // keys per workgroup
  constexpr int kBQ = 64;        // query rows per tile
  constexpr int kRowBytes = D * 2;
  constexpr int kChunks = D / 8;
  constexpr int kDc = D / 16;
  constexpr int kHalves = D / dkdv_cols<D>();  // column halves of dK / dV (one per workgroup)
  constexpr int kDt = dkdv_cols<D>() / 32;     // 32-column output tiles of this workgroup
  constexpr int kTileBytes = kBQ * kRowBytes;
  constexpr int kVecBytes = kBQ * 4;
  constexpr int kBufBytes = 2 * kTileBytes + 2 * kVecBytes;  // Q, dO, lse2, D
  constexpr int kLoads = kTileBytes / 1024 / kNW;
  static_assert(kLoads * 1024 * kNW == kTileBytes, "tile must split evenly over waves");
  static_assert(kBQ == 64, "one dword load per lane fills a per-row slice");
  constexpr int kBitmapBytes = MODE == kMask ? kMaxQBlocks / 8 : 0;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kBufBytes + kBitmapBytes];

  int tile, unit;
  decode(p, false, tile, unit);  // causal: low key blocks (most query tiles) first
  const int half = unit % kHalves;  // the dK / dV columns 32 kDt half .. of this workgroup
  const int b = unit / kHalves / p.hkv;
  const int kvh = unit / kHalves % p.hkv;
  int64_t tok0 = 0;
  int len = p.seqlen;
  if (p.cu) {
    tok0 = p.cu[b];
    len = min(p.cu[b + 1] - p.cu[b], p.seqlen);  // seqlen bounds every length
  }
  const int k0 = tile * kBK;
  if (k0 >= len) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int j16 = lane & 15;

  const uint16_t *kg = p.k + (p.cu ? tok0 * p.k_ss : (int64_t)b * p.k_sb) + (int64_t)kvh * p.k_sh;
  const uint16_t *vg = p.v + (p.cu ? tok0 * p.v_ss : (int64_t)b * p.v_sb) + (int64_t)kvh * p.v_sh;
  const uint16_t *qbase = p.q + (p.cu ? tok0 * p.q_ss : (int64_t)b * p.q_sb);
  const uint16_t *gbase = p.g + (p.cu ? tok0 * p.g_ss : (int64_t)b * p.g_sb);

  // ---- query iteration space.  Query blocks of 128 that may see this key
  // block: all, those at or below the diagonal (causal), or those whose mask
  // row has this block's bit set; each is visited for every query head of the
  // group, as two tiles of 64 rows.  Step it = (block j, head hh, half sub)
  // with it = (j * group + hh) * 2 + sub.
  const int n_qblk = (len + kListBlock - 1) / kListBlock;
  const int qb_lo = CAUSAL ? tile : 0;
  uint32_t *bitmap = reinterpret_cast<uint32_t *>(smem + 2 * kBufBytes);
  int n_vis;
  if (MODE == kMask) {
    // column bitmap: bit qb set when row qb of the mask has this key block's bit
    const uint32_t *mcol = p.mask + b * p.mask_ss + kvh * p.mask_sh + (tile >> 5);
    for (int base = 0; base < n_qblk; base += 64 * kNW) {
      const int qb = base + tid;
      bool bit = false;
      if (qb < n_qblk && qb >= qb_lo) bit = (mcol[(int64_t)qb * p.mask_words] >> (tile & 31)) & 1u;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(bit);
      if (lane == 0 && base + wave * 64 < n_qblk) {
        bitmap[(base + wave * 64) >> 5] = (uint32_t)bal;
        if (base + wave * 64 + 32 < n_qblk) bitmap[((base + wave * 64) >> 5) + 1] = (uint32_t)(bal >> 32);
      }
    }
    __syncthreads();
    n_vis = 0;
    for (int w = 0; w < (n_qblk + 31) >> 5; ++w) n_vis += __builtin_popcount(bitmap[w]);
  } else {
    n_vis = n_qblk - qb_lo;
  }
  const int n_iter = n_vis * p.group * 2;
  int c_w = -1;         // bitmap word being walked
  uint32_t c_bits = 0;  // its set bits not yet visited
  int c_blk = qb_lo - 1;
  // query row start and head of step `it` (called for it = 0, 1, 2, ... in
  // order)
  auto q_start = [&](int it, int &head) -> int {
    const int sub = it & 1;
    const int hh = (it >> 1) % p.group;
    if ((it >> 1) % p.group == 0 && sub == 0) {
      if (MODE == kMask) {
        while (c_bits == 0) c_bits = bitmap[++c_w];
        c_blk = 32 * c_w + __builtin_ctz(c_bits);
        c_bits &= c_bits - 1u;
      } else {
        ++c_blk;
      }
    }
    head = kvh * p.group + hh;
    // a tile past the end of the sequence is loaded from the last row and
    // computed fully masked, so the step has no branch around the
    // accumulators (which would make the compiler copy them)
    return c_blk * kListBlock + sub * kBQ;
  };

  // ---- direct global -> LDS loads of one query tile: Q and dO rows (dual
  // layout) and the workspace's lse2 and D of the same rows (waves 0 and 1,
  // one dword per lane); rows past the end re-read the last row
  // (byte offsets of this lane's loads within a tile's rows; row of load n:
  // lrow0 + n * kRowStep)
  constexpr int kRowStep = 64 / kChunks;
  static_assert(64 % kChunks == 0, "a wave-wide load covers whole rows");
  uint32_t qoff[kLoads], goff[kLoads];
  const int slot_byte0 = wave * kLoads * 1024;
  const int lrow0 = (wave * kLoads * 64 + lane) / kChunks;
  const uint32_t q_ssb = (uint32_t)p.q_ss * 2u, g_ssb = (uint32_t)p.g_ss * 2u;  // row strides in bytes
#pragma unroll
  for (int n = 0; n < kLoads; ++n) {
    const int slot = (wave * kLoads + n) * 64 + lane;
    const int r = slot / kChunks, pc = slot % kChunks;
    qoff[n] = (uint32_t)r * q_ssb + (uint32_t)(pc ^ L::f(r)) * 16u;
    goff[n] = (uint32_t)r * g_ssb + (uint32_t)(pc ^ L::f(r)) * 16u;
  }
  // Loads of the query tile at q0 of `head` into buffer buf: Q and dO rows
  // (unless `rows_deferred`: a whole tile whose rows the caller issues
  // itself, one load at a time) and the lse2 / D values.
  auto issue = [&](int buf, int q0, int head, bool rows_deferred = false) {
    char *bq = smem + buf * kBufBytes;
    const char *qt = reinterpret_cast<const char *>(qbase + (int64_t)head * p.q_sh + (int64_t)q0 * p.q_ss);
    const char *gt = reinterpret_cast<const char *>(gbase + (int64_t)head * p.g_sh + (int64_t)q0 * p.g_ss);
    const int rows_left = len - q0;
    if (rows_deferred) {
    } else if (rows_left >= kBQ)
      issue_pair_full<kLoads>(bq + slot_byte0, bq + kTileBytes + slot_byte0, qt, gt, qoff, goff);
    else
      issue_pair<kLoads, kRowStep>(bq + slot_byte0, bq + kTileBytes + slot_byte0, qt, gt, qoff, goff, lrow0,
                                   q_ssb, g_ssb, rows_left);
    if (wave < 2) {
      const int row = q0 + min(lane, rows_left - 1);
      const float *src = (wave == 0 ? p.ws_lse2 : p.ws_d) + ws_index(p, b, head, row);
      issue_dwords(bq + 2 * kTileBytes + wave * kVecBytes, src);
    }
  };

  int head_cur = 0;
  int q_cur = 0;
  if (n_iter > 0) {
    q_cur = q_start(0, head_cur);
    issue(0, q_cur, head_cur);
  }

  // ---- K and V rows of this wave's 32 keys as MFMA B operands (lane l32 =
  // key, head-dim values 16 dc + 8 hi .. +7); keys past the end read as zero
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;
  bf16x8_t kreg[kDc], vreg[kDc];
#pragma unroll
  for (int dc = 0; dc < kDc; ++dc) {
    uint4_t x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (key < len) {
      x = ld_global16(kg + (int64_t)key * p.k_ss + dc * 16 + hi * 8);
      y = ld_global16(vg + (int64_t)key * p.v_ss + dc * 16 + hi * 8);
    }
    kreg[dc] = __builtin_bit_cast(bf16x8_t, x);
    vreg[dc] = __builtin_bit_cast(bf16x8_t, y);
  }

  floatx16_t dk[kDt], dv[kDt];
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk[dt][i] = 0.f;
      dv[dt][i] = 0.f;
    }

  // per-lane LDS offsets: row-wise reads of Q and dO (row l32, chunk
  // 2 dc + hi) and transpose reads (rows 4 hi + j16/4 and 8 more, the 4
  // columns at 32 dt + 16 (l32/16) + 4 (j16%4))
  uint32_t raddr[kDc];
  uint32_t ta[kDt], tb[kDt];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_char_t *)smem;
#pragma unroll
  for (int dc = 0; dc < kDc; ++dc) {
    raddr[dc] = smem_lds + L::at(l32, 2 * dc + hi);
    asm volatile("" : "+v"(raddr[dc]));
  }
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt) {
    const int ch = 4 * (half * kDt + dt) + 2 * (l32 >> 4) + ((j16 & 3) >> 1);
    ta[dt] = smem_lds + L::at(4 * hi + (j16 >> 2), ch) + (j16 & 1) * 8;
    tb[dt] = smem_lds + L::at(8 + 4 * hi + (j16 >> 2), ch) + (j16 & 1) * 8;
    asm volatile("" : "+v"(ta[dt]));
    asm volatile("" : "+v"(tb[dt]));
  }

  // One query tile per step; the LDS buffer alternates at run time, so the
  // loop body (and the register assignment of the accumulators) exists once.
  auto step = [&](const int it, const int buf) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    int q_nxt = 0, head_nxt = 0;
    // a whole next tile has its Q / dO row loads spread over the first
    // half's S / dP MFMAs (their issue would otherwise hold up the matrix
    // core after the barrier); a partial one is issued here
    bool spread = false;
    if (it + 1 < n_iter) {
      q_nxt = q_start(it + 1, head_nxt);
      spread = len - q_nxt >= kBQ;
      issue(1 - buf, q_nxt, head_nxt, spread);
    }
    const char *const qt_n =
        reinterpret_cast<const char *>(qbase + (int64_t)head_nxt * p.q_sh + (int64_t)q_nxt * p.q_ss);
    const char *const gt_n =
        reinterpret_cast<const char *>(gbase + (int64_t)head_nxt * p.g_sh + (int64_t)q_nxt * p.g_ss);
    char *const bq_n = smem + (1 - buf) * kBufBytes + slot_byte0;
    const int q0 = q_cur;
    q_cur = q_nxt;
    const int boff = buf * kBufBytes;
    // The tile's two halves of 32 query rows are software-pipelined so that
    // the exp2 / dS VALU work of one half runs between the MFMAs of the other
    // (one wave per SIMD: nothing else would fill the matrix core meanwhile):
    //   S, dP of half 0 | S, dP of half 1 + VALU of half 0 |
    //   dV, dK of half 0 + VALU of half 1 | dV, dK of half 1.
    floatx16_t s[2], dp[2];
    bf16x8_t pb[2][2], dsb[2][2];
    typedef __attribute__((ext_vector_type(4))) float f32x4_t;
    f32x4_t l4[2][4], d4[2][4];
    // lse2 and D of this lane's 16 rows of half h (register i: row 8 (i/4) +
    // 4 hi + i%4), by inline-assembly reads like the operand rings (a plain
    // load would make the compiler wait for every LDS read in flight at the
    // first use).  Read early (head_dim 128), they need no wait of their own:
    // the half's VALU uses S of that half, whose last MFMA follows the
    // lgkmcnt(0) that ends its phase, which comes after these reads (LDS
    // reads complete in order).  Read late (head_dim 64), ld_wait ties them
    // to a wait of their own.
    const uint32_t ld_base = smem_lds + boff + 2 * kTileBytes + 16 * hi;
    auto load_ld = [&](auto H) __attribute__((always_inline)) {
      constexpr int h = decltype(H)::value;
      static_for<4>([&](auto G) {
        constexpr int g4 = decltype(G)::value;
        l4[h][g4] = __builtin_bit_cast(f32x4_t, ld_b128<(32 * h + 8 * g4) * 4>(ld_base));
        d4[h][g4] = __builtin_bit_cast(f32x4_t, ld_b128<(kBQ + 32 * h + 8 * g4) * 4>(ld_base));
      });
    };
    auto ld_wait = [&](auto H) __attribute__((always_inline)) {
      constexpr int h = decltype(H)::value;
      f32x4_t(&lh)[4] = l4[h];
      f32x4_t(&dh)[4] = d4[h];
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(lh[0]), "+v"(lh[1]), "+v"(lh[2]), "+v"(lh[3]), "+v"(dh[0]), "+v"(dh[1]), "+v"(dh[2]),
                     "+v"(dh[3]));
    };
    // Register i of half h holds query row qh0 + 4 hi + r, r = 8 (i/4) + i%4
    // (a compile-time offset): the row is visible to this lane's key when
    // r >= key - (qh0 + 4 hi) (causal) and r < len - (qh0 + 4 hi)
    int rlo[2], rhi[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r0 = q0 + 32 * h + 4 * hi;
      rlo[h] = key - r0;
      rhi[h] = len - r0;
    }
    // VALU of element i (of 16) of half h: P = 2^(c s - lse2), dS = P (dP - D),
    // spread over the MFMA steps of the other half; no mask here
    auto valu = [&](auto H, auto I) __attribute__((always_inline)) {
      constexpr int h = decltype(H)::value, i = decltype(I)::value;
      constexpr int g4 = i / 4, e = i % 4;
      const float lv = l4[h][g4][e];
      const float dv4 = d4[h][g4][e];
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][i], p.c, -lv));
      pb[h][i >> 3][i & 7] = (__bf16)pv;
      dsb[h][i >> 3][i & 7] = (__bf16)(pv * (dp[h][i] - dv4));
    };
    // A half whose rows reach past the end, or (causal) precede some of this
    // wave's keys, then has P and dS zeroed where the row is past the end or
    // before the lane's key (a uniform branch, taken on the diagonal and the
    // tail only; evaluating the mask inside the spread VALU would cost two
    // compares and a select per element on every half).  Patching, rather
    // than forming the half again, keeps the spread VALU's results live on
    // both paths, so the compiler cannot sink them below the branch.
    auto fixup = [&](auto H) __attribute__((always_inline)) {
      constexpr int h = decltype(H)::value;
      const int qh0 = q0 + 32 * h;
      if ((qh0 + 32 > len) || (CAUSAL && qh0 < kw0 + 31)) {
        asm volatile("; masked half");
        static_for<16>([&](auto I) {
          constexpr int i = decltype(I)::value, r = 8 * (i / 4) + i % 4;
          if (r >= rhi[h] || (CAUSAL && r < rlo[h])) {
            pb[h][i >> 3][i & 7] = (__bf16)0.f;
            dsb[h][i >> 3][i & 7] = (__bf16)0.f;
          }
        });
      }
    };
    // this tile's buffer: row-wise read addresses of Q (dO kTileBytes on)
    uint32_t rb[kDc];
#pragma unroll
    for (int dc = 0; dc < kDc; ++dc) rb[dc] = raddr[dc] + boff;
    // S = Q K^T and dP = dO V^T of half h (32 query rows x 32 keys; lane =
    // key), operand reads kRing MFMAs ahead with exact waits, S and dP
    // alternating; the VALU of half hv (if hv >= 0) spread over the steps
    auto sdp = [&](auto H, auto HV) __attribute__((always_inline)) {
      constexpr int h = decltype(H)::value, hv = decltype(HV)::value;
      constexpr int kRing = 4;
      constexpr int kSteps = 2 * kDc;  // step i: dc = i / 2, Q (even) or dO (odd)
      // VALU elements per step (kPer on every kStride-th step)
      constexpr int kPer = kSteps >= 16 ? 1 : 16 / kSteps;
      constexpr int kStride = kSteps >= 16 ? kSteps / 16 : 1;
      static_assert(2 * kLoads <= kSteps, "the next tile's row loads fit in the first half's steps");
      bf16x8_t ring[kRing];
      static_for<kRing>([&](auto I) {
        constexpr int i = decltype(I)::value;
        ring[i] = ld_b128<h * 32 * kRowBytes + (i & 1) * kTileBytes>(rb[i >> 1]);
      });
      static_for<kSteps>([&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr int dc = i >> 1;
        lgkm_wait<(kSteps - 1 - i < kRing - 1 ? kSteps - 1 - i : kRing - 1)>(ring[i % kRing]);
        if constexpr (i & 1) {
          if constexpr (dc == 0)
            dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], vreg[dc], floatx16_t{}, 0, 0, 0);
          else
            dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], vreg[dc], dp[h], 0, 0, 0);
        } else {
          if constexpr (dc == 0)
            s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], kreg[dc], floatx16_t{}, 0, 0, 0);
          else
            s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], kreg[dc], s[h], 0, 0, 0);
        }
        if constexpr (i + kRing < kSteps) {
          constexpr int j = i + kRing;
          ring[i % kRing] = ld_b128<h * 32 * kRowBytes + (j & 1) * kTileBytes>(rb[j >> 1]);
        }
        if constexpr (h == 0 && i < 2 * kLoads) {
          // load i / 2 of the next tile's Q (even i) or dO (odd i) rows
          constexpr int n = i >> 1;
          if (spread) {
            if constexpr (i & 1)
              issue_one<n>(bq_n + kTileBytes, gt_n, goff);
            else
              issue_one<n>(bq_n, qt_n, qoff);
          }
        }
        if constexpr (hv >= 0 && i % kStride == 0)
          static_for<kPer>([&](auto E) {
            valu(HV, std::integral_constant<int, (i / kStride) * kPer + decltype(E)::value>{});
          });
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // dV += P^T dO and dK += dS^T Q of half h.  B operands by transpose reads
    // of rows 16 c + 8 (e/4) + 4 hi + e%4 of the half (the k order of P); the
    // reads run kRing MFMAs ahead; the VALU of half hv (if hv >= 0) spread
    // over the steps
    auto dvdk = [&](auto H, auto HV) __attribute__((always_inline)) {
      constexpr int h = decltype(H)::value, hv = decltype(HV)::value;
      const int hoff = boff + h * 32 * kRowBytes;  // row 0 of this half in the Q tile
      uint32_t ha[kDt], hb[kDt];
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        ha[dt] = ta[dt] + hoff;
        hb[dt] = tb[dt] + hoff;
      }
      constexpr int kRing = 4;
      constexpr int kSteps = kDt * 2 * 2;  // step i: dO (even) or Q (odd); (dt, c) = i / 2
      constexpr int kPer = 16 / kSteps;
      bf16x8_t ring[kRing];
      static_for<kRing>([&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr int dt = (i >> 1) % kDt, c = (i >> 1) / kDt;
        constexpr int off = c * 16 * kRowBytes + ((i & 1) ? 0 : kTileBytes);
        ring[i] = tr_pair2<off>(ha[dt], hb[dt]);
      });
      static_for<kSteps>([&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr int dt = (i >> 1) % kDt, c = (i >> 1) / kDt;
        lgkm_wait<2 * (kSteps - 1 - i < kRing - 1 ? kSteps - 1 - i : kRing - 1)>(ring[i % kRing]);
        if constexpr (i & 1)
          dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsb[h][c], ring[i % kRing], dk[dt], 0, 0, 0);
        else
          dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pb[h][c], ring[i % kRing], dv[dt], 0, 0, 0);
        if constexpr (i + kRing < kSteps) {
          constexpr int j = i + kRing;
          constexpr int dtj = (j >> 1) % kDt, cj = (j >> 1) / kDt;
          constexpr int offj = cj * 16 * kRowBytes + ((j & 1) ? 0 : kTileBytes);
          ring[i % kRing] = tr_pair2<offj>(ha[dtj], hb[dtj]);
        }
        if constexpr (hv >= 0)
          static_for<kPer>([&](auto E) { valu(HV, std::integral_constant<int, i * kPer + decltype(E)::value>{}); });
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using CN = std::integral_constant<int, -1>;
    // (at head_dim 128 the wave has registers to spare for both halves'
    // values at once; at 64 they are read just before their half's VALU)
    constexpr bool kEarly = D == 128;
    if constexpr (kEarly) load_ld(C0{});
    sdp(C0{}, CN{});
    if constexpr (kEarly) {
      load_ld(C1{});
    } else {
      load_ld(C0{});
      ld_wait(C0{});
    }
    sdp(C1{}, C0{});
    fixup(C0{});
    if constexpr (!kEarly) {
      load_ld(C1{});
      ld_wait(C1{});
    }
    dvdk(C0{}, C1{});
    fixup(C1{});
    dvdk(C1{}, CN{});
  };
  for (int it = 0; it < n_iter; ++it) step(it, it & 1);

  // ---- epilogue: dK = scale * acc, dV = acc in bf16.  Register i of tile dt
  // holds key 8 (i/4) + 4 hi + i%4 of the wave, head-dim column 32 dt + l32.
  uint16_t *dkg = p.dk + (p.cu ? tok0 * p.dk_ss : (int64_t)b * p.dk_sb) + (int64_t)kvh * p.dk_sh;
  uint16_t *dvg = p.dv + (p.cu ? tok0 * p.dv_ss : (int64_t)b * p.dv_sb) + (int64_t)kvh * p.dv_sh;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kr = kw0 + (i >> 2) * 8 + hi * 4 + (i & 3);
    if (kr < len) {
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        const __bf16 xk = (__bf16)(dk[dt][i] * p.scale);
        const __bf16 xv = (__bf16)dv[dt][i];
        const int col = 32 * (half * kDt + dt) + l32;
        dkg[(int64_t)kr * p.dk_ss + col] = __builtin_bit_cast(uint16_t, xk);
        dvg[(int64_t)kr * p.dv_ss + col] = __builtin_bit_cast(uint16_t, xv);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
size_t ws_entries(const attn_tensor_t *q) {
  return (size_t)q->heads * (size_t)q->batch * (size_t)q->seqlen;
}

// Argument checks of attn_bwd other than the workspace.
int validate_bwd_args(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                      const attn_tensor_t *out, const attn_tensor_t *dout, const float *lse,
                      const int32_t *cu, int causal, float scale, const attn_block_mask_t *mask,
                      const attn_tensor_t *dq, const attn_tensor_t *dk, const attn_tensor_t *dv) {
  if (!dout || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
  // q, k, v, out; then dout and dq like out, dk and dv like k and v
  int st = mask ? attn_fwd_mask_validate(q, k, v, cu, causal, scale, mask, out)
                : attn_fwd_validate(q, k, v, cu, causal, scale, nullptr, out);
  if (st != ATTN_OK) return st;
  st = attn_fwd_validate(q, k, v, cu, causal, scale, nullptr, dout);
  if (st != ATTN_OK) return st;
  st = attn_fwd_validate(q, dk, dv, cu, causal, scale, nullptr, dq);
  if (st != ATTN_OK) return st;
  if (dk->heads != k->heads) return ATTN_ERR_INVALID_ARG;
  // the dK/dV kernel addresses the rows of a Q or dO tile with 32-bit byte
  // offsets from the tile's first row, as every kernel does for K and V
  for (const attn_tensor_t *t : {q, dout})
    if (t->stride_seq < 0 || t->stride_seq >= kMaxRowStride) return ATTN_ERR_UNSUPPORTED;
  const bool empty = q->batch == 0 || q->seqlen == 0;
  if (empty) return ATTN_OK;
  if (!lse) return ATTN_ERR_INVALID_ARG;
  if (mask && (q->seqlen + kListBlock - 1) / kListBlock > kMaxQBlocks) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

int validate_bwd(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                 const attn_tensor_t *out, const attn_tensor_t *dout, const float *lse,
                 const int32_t *cu, int causal, float scale, const attn_block_mask_t *mask,
                 const attn_tensor_t *dq, const attn_tensor_t *dk, const attn_tensor_t *dv,
                 const void *ws, size_t ws_bytes) {
  const int st = validate_bwd_args(q, k, v, out, dout, lse, cu, causal, scale, mask, dq, dk, dv);
  if (st != ATTN_OK) return st;
  if (q->batch == 0 || q->seqlen == 0) return ATTN_OK;
  if (!ws) return ATTN_ERR_INVALID_ARG;
  if (ws_bytes < 2 * sizeof(float) * ws_entries(q)) return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)ws & 15u) != 0) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

template <int D, bool CAUSAL, int MODE>
int launch_pair(BwdParams p, hipStream_t s) {
  const int n_tiles = (p.seqlen + 127) / 128;
  // dQ: one workgroup per 128-row query tile of each (sequence, query head)
  p.n_tiles = n_tiles;
  p.n_units = p.batch * p.hq;
  p.unit_group = p.group;
  p.xcd_remap = (p.n_units % (8 * p.group)) == 0 ? 1 : 0;
  {
    void *args[] = {&p};
    const hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void *>(&attn_bwd_dq_kernel<D, CAUSAL, MODE>),
        dim3((unsigned)((int64_t)n_tiles * p.n_units)), dim3(256), args, 0, s);
    if (e != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  // dK/dV: one workgroup per 128-key block of each (sequence, KV head) and
  // column half (head_dim 256), the halves of one KV head on one XCD
  const int halves = D / dkdv_cols<D>();
  p.n_units = p.batch * p.hkv * halves;
  p.unit_group = halves;
  p.xcd_remap = (p.n_units % (8 * halves)) == 0 ? 1 : 0;
  {
    void *args[] = {&p};
    const hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void *>(&attn_bwd_dkdv_kernel<D, CAUSAL, MODE>),
        dim3((unsigned)((int64_t)n_tiles * p.n_units)), dim3(256), args, 0, s);
    if (e != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

template <int D>
int launch_d(const BwdParams &p, bool causal, bool masked, hipStream_t s) {
  if (masked) return causal ? launch_pair<D, true, kMask>(p, s) : launch_pair<D, false, kMask>(p, s);
  return causal ? launch_pair<D, true, kDense>(p, s) : launch_pair<D, false, kDense>(p, s);
}

}  // namespace

extern "C" size_t attn_bwd_workspace_size(const attn_tensor_t *q) {
  if (!q || q->batch <= 0 || q->seqlen <= 0 || q->heads <= 0) return 0;
  return 2 * sizeof(float) * ws_entries(q);
}

extern "C" int attn_bwd_validate(const attn_tensor_t *q, const attn_tensor_t *k,
                                 const attn_tensor_t *v, const attn_tensor_t *out,
                                 const attn_tensor_t *dout, const float *lse,
                                 const int32_t *cu_seqlens, int causal, float scale,
                                 const attn_block_mask_t *mask, const attn_tensor_t *dq,
                                 const attn_tensor_t *dk, const attn_tensor_t *dv,
                                 const void *workspace, size_t workspace_bytes) {
  return validate_bwd(q, k, v, out, dout, lse, cu_seqlens, causal, scale, mask, dq, dk, dv,
                      workspace, workspace_bytes);
}

namespace {

// Both kernels of the backward, with the per-row workspace at `workspace`
// (already validated).
int run_bwd(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
            const attn_tensor_t *out, const attn_tensor_t *dout, const float *lse,
            const int32_t *cu_seqlens, int causal, float scale, const attn_block_mask_t *mask,
            attn_tensor_t *dq, attn_tensor_t *dk, attn_tensor_t *dv, void *workspace,
            void *stream) {
  BwdParams p;
  p.q = static_cast<const uint16_t *>(q->data);
  p.k = static_cast<const uint16_t *>(k->data);
  p.v = static_cast<const uint16_t *>(v->data);
  p.o = static_cast<const uint16_t *>(out->data);
  p.g = static_cast<const uint16_t *>(dout->data);
  p.lse = lse;
  p.dq = static_cast<uint16_t *>(dq->data);
  p.dk = static_cast<uint16_t *>(dk->data);
  p.dv = static_cast<uint16_t *>(dv->data);
  p.ws_lse2 = static_cast<float *>(workspace);
  p.ws_d = p.ws_lse2 + ws_entries(q);
  p.q_sb = q->stride_batch; p.q_ss = q->stride_seq; p.q_sh = q->stride_head;
  p.k_sb = k->stride_batch; p.k_ss = k->stride_seq; p.k_sh = k->stride_head;
  p.v_sb = v->stride_batch; p.v_ss = v->stride_seq; p.v_sh = v->stride_head;
  p.o_sb = out->stride_batch; p.o_ss = out->stride_seq; p.o_sh = out->stride_head;
  p.g_sb = dout->stride_batch; p.g_ss = dout->stride_seq; p.g_sh = dout->stride_head;
  p.dq_sb = dq->stride_batch; p.dq_ss = dq->stride_seq; p.dq_sh = dq->stride_head;
  p.dk_sb = dk->stride_batch; p.dk_ss = dk->stride_seq; p.dk_sh = dk->stride_head;
  p.dv_sb = dv->stride_batch; p.dv_ss = dv->stride_seq; p.dv_sh = dv->stride_head;
  p.cu = cu_seqlens;
  p.mask = mask ? mask->bits : nullptr;
  p.mask_ss = mask ? mask->stride_seq : 0;
  p.mask_sh = mask ? mask->stride_head : 0;
  p.mask_words = mask ? mask->words_per_row : 0;
  p.batch = q->batch;
  p.seqlen = q->seqlen;
  p.hq = q->heads;
  p.hkv = k->heads;
  p.group = q->heads / k->heads;
  p.n_tiles = p.n_units = p.unit_group = p.xcd_remap = 0;  // set per kernel at launch
  p.c = scale * kLog2e;
  p.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q->head_dim == 64) return launch_d<64>(p, causal != 0, mask != nullptr, s);
  if (q->head_dim == 256) return launch_d<256>(p, causal != 0, mask != nullptr, s);
  return launch_d<128>(p, causal != 0, mask != nullptr, s);
}

// ---------------------------------------------------------------------------
// Static scratch of attn_bwd_noalloc: the per-row workspace of the backward
// in a fixed device array, for callers that cannot allocate.  In host code
// `scratch` names a host-side stand-in, not device memory, so its device
// address is taken once per device with hipGetSymbolAddress (each device
// holds its own copy) and only that address is handed to the kernels.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) char scratch[ATTN_BWD_SCRATCH_BYTES];

namespace {

// Device address of the current device's scratch (taken on the first call on
// that device), or null if it cannot be obtained.
void *scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// The mask row of one query block from its block list: cleared, then one
// bit per listed id in range, in LDS; written out in full.  One workgroup
// per query block.
constexpr int kMaxMaskWords = kMaxQBlocks / 32;
__global__ __launch_bounds__(256) void list_to_mask_kernel(const int32_t *row_ptr, const int32_t *col_idx,
                                                           int n_kv_blocks, uint32_t *mask, int words) {
  __shared__ uint32_t row[kMaxMaskWords];
  const int qb = blockIdx.x;
  for (int w = threadIdx.x; w < words; w += 256) row[w] = 0u;
  __syncthreads();
  const int e0 = row_ptr[qb], e1 = row_ptr[qb + 1];
  for (int e = e0 + (int)threadIdx.x; e < e1; e += 256) {
    const int kb = col_idx[e];
    if (kb >= 0 && kb < n_kv_blocks) atomicOr(&row[kb >> 5], 1u << (kb & 31));
  }
  __syncthreads();
  for (int w = threadIdx.x; w < words; w += 256) mask[(int64_t)qb * words + w] = row[w];
}

}  // namespace

extern "C" int attn_block_list_to_mask(const attn_block_list_t *list, int n_kv_blocks, uint32_t *mask,
                                       int mask_words, void *stream) {
  if (!list || n_kv_blocks < 0 || list->num_q_blocks < 0 || mask_words < 0) return ATTN_ERR_INVALID_ARG;
  if (list->block_q != kListBlock || list->block_k != kListBlock) return ATTN_ERR_UNSUPPORTED;
  if (n_kv_blocks > kMaxQBlocks) return ATTN_ERR_UNSUPPORTED;
  if (mask_words < (n_kv_blocks + 31) / 32 || mask_words > kMaxMaskWords) return ATTN_ERR_INVALID_ARG;
  if (list->num_q_blocks == 0) return ATTN_OK;
  if (!list->row_ptr || !list->col_idx || !mask || mask_words == 0) return ATTN_ERR_INVALID_ARG;
  const int32_t *row_ptr = list->row_ptr, *col_idx = list->col_idx;
  void *args[] = {&row_ptr, &col_idx, &n_kv_blocks, &mask, &mask_words};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&list_to_mask_kernel),
                                       dim3((unsigned)list->num_q_blocks), dim3(256), args, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" int attn_bwd(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                        const attn_tensor_t *out, const attn_tensor_t *dout, const float *lse,
                        const int32_t *cu_seqlens, int causal, float scale,
                        const attn_block_mask_t *mask, attn_tensor_t *dq, attn_tensor_t *dk,
                        attn_tensor_t *dv, void *workspace, size_t workspace_bytes,
                        void *stream) {
  const int st = validate_bwd(q, k, v, out, dout, lse, cu_seqlens, causal, scale, mask, dq, dk,
                              dv, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  if (q->batch == 0 || q->seqlen == 0) return ATTN_OK;
  return run_bwd(q, k, v, out, dout, lse, cu_seqlens, causal, scale, mask, dq, dk, dv, workspace,
                 stream);
}

extern "C" int attn_bwd_noalloc(const attn_tensor_t *q, const attn_tensor_t *k,
                                const attn_tensor_t *v, const attn_tensor_t *out,
                                const attn_tensor_t *dout, const float *lse,
                                const int32_t *cu_seqlens, int causal, float scale,
                                const attn_block_mask_t *mask, attn_tensor_t *dq,
                                attn_tensor_t *dk, attn_tensor_t *dv, void *stream) {
  const int st = validate_bwd_args(q, k, v, out, dout, lse, cu_seqlens, causal, scale, mask, dq,
                                   dk, dv);
  if (st != ATTN_OK) return st;
  if (q->batch == 0 || q->seqlen == 0) return ATTN_OK;
  if (2 * sizeof(float) * ws_entries(q) > (size_t)ATTN_BWD_SCRATCH_BYTES) return ATTN_ERR_TOO_LARGE;
  void *ws = scratch_address();
  if (!ws) return ATTN_ERR_LAUNCH;
  return run_bwd(q, k, v, out, dout, lse, cu_seqlens, causal, scale, mask, dq, dk, dv, ws, stream);
}
