// attn_entmax.hip — alpha-entmax attention forward for AMD Instinct MI355X (gfx950).
//
// alpha-entmax replaces the softmax normaliser by a threshold tau found by
// root finding (AdaSplash-2 explainer, technical summary section 1):
//   p_j = [(alpha-1) z_j - tau]_+^(1/(alpha-1)),  sum_j p_j = 1,  O = sum_j p_j v_j.
// Following the explainer's section 2, one workgroup (128 query rows of one
// (sequence, query head), four wave64s of 32 rows) makes these passes over
// the keys it may see, each streaming 64-key K tiles through double-buffered
// LDS with direct global-to-LDS loads and forming the transposed score tile
// S^T = K Q^T with 32x32x16 bf16 MFMAs (lane = query row, as in the softmax
// kernel):
//   1. the row maximum m and, in the same pass, a histogram of the scores
//      in the window [m - W, m], W = 1/(alpha-1) (only those can carry
//      weight): kBins bins in LDS of width W/(kBins-1) on a fixed grid,
//      kept per lane as a ring that follows the running maximum; each score
//      counts at its bin's lower edge, so the root tau_h of the histogram's
//      mass equation is a lower bound of the true tau; each lane finds the
//      bin that holds it and solves inside that bin;
//   2. up to n_iter refinement passes (fewer once every row of the workgroup
//      has converged or taken its last step), each forming the power sums the update needs
//      at the current tau and taking one step of the hybrid solver (Halley
//      for alpha <= 1.5, Newton for alpha <= 2, a secant through the bracket
//      ends (regula falsi, Illinois rule) above), with a
//      bisection step whenever the update leaves the bracket [lo, hi] kept
//      from the signs seen so far; every pass also marks, in an LDS
//      bit-packed block mask, each 128-key block whose scores can clear the
//      bracket's lower end at the start of the pass (so every block with a
//      non-zero weight at the final tau is marked); above alpha = 2 the
//      first of them also gathers each row's few keys above the bracket's
//      lower end and solves the mass equation on them exactly;
//   3. the output pass, which visits only the marked blocks (walking the
//      mask's set bits), forms p in registers and accumulates O^T += V^T P^T
//      with V^T from LDS transpose reads; O is divided by sum p.
// tau (fp32) and the bit-packed block mask can be written out.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn_common.h"
#include "attn_fwd.h"

namespace {

using namespace attn_detail;

constexpr int kBins = 32;       // histogram bins per row
constexpr int kMaxKBlocks = 16384;  // key blocks a mask row holds in LDS

struct EntParams {
  const uint16_t *q, *k, *v;
  uint16_t *o;
  float *tau;          // [B, Hq, S] or null
  float *tau_init;     // [B, Hq, S] or null: the histogram bound tau_h
  uint32_t *mask;      // [B, Hq, n_qblk, mask_words] or null
  int mask_words;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int batch, seqlen, hq, group, n_tiles, n_iter, causal;
  float scale, alpha;
};

// The weights' exponent e = 1/(alpha-1): alpha = 2 (sparsemax) gives e = 1
// and alpha = 1.5 gives e = 2, where u^e and the power sums of the solver
// need no transcendental; every other alpha goes through exp2/log2.
enum { kPowGeneral = 0, kPowLinear = 1, kPowSquare = 2 };

// u^e for u > 0 (0 otherwise)
// (products without a branch; the transcendental pair behind one, which
// skips it whenever no lane of the wave has u > 0 -- most scores, since only
// those within 1/(alpha-1) of the row max can carry weight)
template <int PK>
__device__ __forceinline__ float powpos(float u, float e) {
  if constexpr (PK == kPowLinear) {
    return fmaxf(u, 0.f);
  } else if constexpr (PK == kPowSquare) {
    const float up = fmaxf(u, 0.f);
    return up * up;
  } else {
    if (!(u > 0.f)) return 0.f;
    return __builtin_amdgcn_exp2f(e * __builtin_amdgcn_logf(u));
  }
}

// LDS read-modify-writes and stores of the histogram and the block mask,
// written as inline assembly: the compiler would order each of its own LDS
// accesses after every direct-to-LDS load in flight (vmcnt(0): it cannot tell
// their addresses apart), which made every tile wait for the next tile's K
// before its first histogram count.  No K/V load writes the histogram or the
// mask; each pass waits for these (lgkmcnt(0)) before its closing barrier.
__device__ __forceinline__ void lds_add_u32(uint32_t addr, uint32_t v) {
  asm volatile("ds_add_u32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_or_b32(uint32_t addr, uint32_t v) {
  asm volatile("ds_or_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_write_b32(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}


// Direct global -> LDS loads of one tile's rows: lane load n reads 16 B at byte
// offset off[n] from the tile's first row t0 (row lrow0 + n * kRowStep of the
// tile) into the n-th 1 KB of `l`.  The offsets are 32-bit (the row strides
// accepted keep a tile's rows within 4 GB of its first) and stay so at the load
// (the empty asm), so each load takes one register offset from a scalar base;
// rows at or past the end of the sequence (rows_left rows remain from t0)
// re-read its last row.
template <int kLoads, int kRowStep, int kTileRows>
__device__ __forceinline__ void issue_rows(char *l, const char *t0, const uint32_t *off, int lrow0,
                                           uint32_t ss_bytes, int rows_left) {
  if (rows_left >= kTileRows) {
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      uint32_t o = off[n];
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(t0 + o, (lds_void_t *)(l + n * 1024), 16, 0, 0);
    }
  } else {
    // r_last: the sequence's last row relative to t0 (negative for a sub-tile
    // of a ragged last block that starts past the end; the base then moves
    // back to it, so that no lane steps back by more than its own row)
    const int r_last = rows_left - 1;
    const int base_row = min(r_last, 0);
    const char *const tb = t0 + (int64_t)base_row * ss_bytes;
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      const int lrow = lrow0 + n * kRowStep;
      const uint32_t back = (uint32_t)(max(lrow - r_last, 0) + base_row);  // 0 <= back <= lrow
      uint32_t o = off[n] - back * ss_bytes;
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(tb + o, (lds_void_t *)(l + n * 1024), 16, 0, 0);
    }
  }
}

// Two workgroups per CU; one at head_dim 256, whose Q rows and O
// accumulators need more than the 256 registers of two waves per SIMD.
template <int D, int PK>
__global__ __launch_bounds__(256, (D == 256 ? 1 : 2)) void attn_entmax_kernel(EntParams p) {
  using L = Lds<D>;
  constexpr int kNW = 4;
  constexpr int kBM = 128;
  constexpr int kBN = D == 256 ? 32 : 64;  // keys per tile (32 at head_dim 256: registers)
  constexpr int kTpb = kListBlock / kBN;    // tiles per 128-key block
  constexpr int kRowBytes = D * 2;
  constexpr int kChunks = D / 8;
  constexpr int kDc = D / 16;
  constexpr int kDt = D / 32;
  constexpr int kKt = kBN / 32;
  constexpr int kTileBytes = kBN * kRowBytes;
  constexpr int kBufBytes = 2 * kTileBytes;  // K then V
  constexpr int kLoads = kTileBytes / 1024 / kNW;
  // Histogram: every lane keeps its own kBins words (a row's two lane halves
  // count separately), word b of lane l of a wave at b * 64 + l of the
  // wave's 8 KB: the lanes of one LDS instruction always hit distinct banks,
  // whatever bins they count, and no word is shared.
  constexpr int kWaveHistBytes = 64 * kBins * 4;
  constexpr int kHistBytes = kNW * kWaveHistBytes;
  constexpr int kMaskBytes = kMaxKBlocks / 8;
  // The passes before the output pass load K only, so the histograms can live
  // in the V halves of the two buffers (two waves' each) when they fit there
  // (they are read into registers before the output pass loads V).
  constexpr bool kHistInV = kTileBytes >= 2 * kWaveHistBytes;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kBufBytes + (kHistInV ? 0 : kHistBytes) + kMaskBytes + 16];
  uint32_t *mbits = reinterpret_cast<uint32_t *>(smem + 2 * kBufBytes + (kHistInV ? 0 : kHistBytes));
  uint32_t *done_flag = mbits + kMaxKBlocks / 32;  // one per wave

  const int n_units = p.batch * p.hq;
  const int rank = blockIdx.x / n_units;
  const int unit = blockIdx.x % n_units;
  const int tile = p.causal ? p.n_tiles - 1 - rank : rank;  // causal: heaviest first
  const int b = unit / p.hq, h = unit % p.hq, kvh = h / p.group;
  const int len = p.seqlen;
  const int q0 = tile * kBM;
  const uint16_t *qg = p.q + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
  const uint16_t *kg = p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
  const uint16_t *vg = p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh;
  uint16_t *og = p.o + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int j16 = lane & 15;
  const int row = wave * 32 + l32;  // row within the workgroup
  const int qrow = q0 + row;
  const bool live = qrow < len;

  const int kv_end = p.causal ? min(len, q0 + kBM) : len;
  const int n_kv = (kv_end + kBN - 1) / kBN;
  const int n_kblk = (kv_end + kListBlock - 1) / kListBlock;
  const float a1 = p.alpha - 1.f;
  const float e = 1.f / a1;
  const float W = e;  // window width 1/(alpha-1)

  // ---- K / V tile loads
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
    koff[n] = (uint32_t)r * k_ssb + (uint32_t)(pc ^ L::kswz(r)) * 16u;
    voff[n] = (uint32_t)r * v_ssb + (uint32_t)L::v_logical_chunk(r, pc) * 16u;
  }
  const char *const kgb = reinterpret_cast<const char *>(kg);
  const char *const vgb = reinterpret_cast<const char *>(vg);
  auto issue = [&](int buf, int kv, bool with_v) {
    char *kb = smem + buf * kBufBytes + slot_byte0;
    issue_rows<kLoads, kRowStep, kBN>(kb, kgb + (int64_t)kv * k_ssb, koff, lrow0, k_ssb, len - kv);
    if (with_v)
      issue_rows<kLoads, kRowStep, kBN>(kb + kTileBytes, vgb + (int64_t)kv * v_ssb, voff, lrow0, v_ssb, len - kv);
  };

  // ---- Q rows (MFMA B operand), zero past the end
  bf16x8_t qreg[kDc];
#pragma unroll
  for (int dc = 0; dc < kDc; ++dc) {
    uint4_t x = {0u, 0u, 0u, 0u};
    if (live) x = ld_global16(qg + (int64_t)qrow * p.q_ss + dc * 16 + hi * 8);
    qreg[dc] = __builtin_bit_cast(bf16x8_t, x);
  }
  // absolute LDS addresses of this lane's K operand reads in buffer 0 (the
  // empty asm keeps each in one register)
  uint32_t kabs[kDc];
#pragma unroll
  for (int dc = 0; dc < kDc; ++dc) {
    kabs[dc] = (uint32_t)(uintptr_t)(lds_char_t *)smem + (uint32_t)L::kq(l32, dc * 2 + hi);
    asm volatile("" : "+v"(kabs[dc]));
  }

  // S^T of one K tile: s[kt][i] is q.k (unscaled: each pass folds the scale
  // into its one FMA per score) of key kv0 + 32 kt + 8 (i/4) + 4 hi + i%4 for
  // this lane's row; keys past kv_end, after the row (causal) or rows past the
  // end get -inf, on the tiles that have such keys (the diagonal and tail)
  auto scores = [&](const int buf_off, int kv0, floatx16_t (&s)[kKt]) {
    {
      // operand reads (K tile at byte buf_off of the LDS) run kRing MFMAs
      // ahead, each waited for exactly (inline-assembly reads: LDS reads
      // complete in order; the compiler would wait for each group of kRing
      // at once); consecutive MFMAs alternate between the kKt accumulators
      // (step i: kt = i % kKt, dc = i / kKt)
      constexpr int kRing = 4;
      constexpr int kSteps = kKt * kDc;
      uint32_t ka[kDc];
#pragma unroll
      for (int dc = 0; dc < kDc; ++dc) ka[dc] = kabs[dc] + (uint32_t)buf_off;
      auto load = [&](auto T) __attribute__((always_inline)) -> bf16x8_t {
        constexpr int t = decltype(T)::value;
        return ld_b128<(t % kKt) * 32 * kRowBytes>(ka[t / kKt]);
      };
      bf16x8_t ring[kRing];
      static_for<kRing>([&](auto T) { ring[decltype(T)::value] = load(T); });
      static_for<kSteps>([&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr int kt = i % kKt, dc = i / kKt;
        lgkm_wait<(kSteps - 1 - i < kRing - 1 ? kSteps - 1 - i : kRing - 1)>(ring[i % kRing]);
        if constexpr (dc == 0)
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], qreg[dc], floatx16_t{}, 0, 0, 0);
        else
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], qreg[dc], s[kt], 0, 0, 0);
        if constexpr (i + kRing < kSteps) ring[i % kRing] = load(std::integral_constant<int, i + kRing>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    const bool need_mask = (kv0 + kBN > kv_end) || (p.causal && kv0 + kBN - 1 > q0 + wave * 32) ||
                           (q0 + wave * 32 + 32 > len);
    if (need_mask) {
      // key kv0 + 4 hi + o (o a compile-time offset) is visible when o <= lim
      const int lim = (live ? (p.causal ? min(qrow, kv_end - 1) : kv_end - 1) : -1) - kv0 - hi * 4;
#pragma unroll
      for (int kt = 0; kt < kKt; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * 32 + (i >> 2) * 8 + (i & 3) > lim) s[kt][i] = -INFINITY;
    }
  };

  // One dense pass over the KV tiles: f(kv0, s) for each.
  auto dense_pass = [&](auto f) {
    issue(0, 0, false);
    for (int it = 0; it < n_kv; ++it) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      if (it + 1 < n_kv) issue((it + 1) & 1, (it + 1) * kBN, false);
      floatx16_t s[kKt];
      scores((it & 1) * kBufBytes, it * kBN, s);
      f(it * kBN, s);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the pass's histogram / mask updates
    __syncthreads();
  };

  // ---- pass 1: the row maximum and the histogram of the window below it,
  // in one pass.  Bins have width bw = W / (kBins - 1) on a grid of integer
  // multiples of bw (bin b holds b bw <= z < (b + 1) bw, b counted from a
  // per-row integer anchor taken at the first tile, so the bin arithmetic
  // stays small); the kBins bins top - kBins + 1 .. top, top the bin of the
  // running maximum, cover the window [m - W, m] whatever m turns out to be.
  // They live in a ring of kBins slots (bin b in slot b mod kBins) per lane,
  // each half of a row counting its own keys (the layout above): when a
  // tile raises top, the slots of the bins that leave the window are cleared
  // for the bins that enter it.  Scores below the window (at the time they
  // are seen, so also at the end) cannot carry weight and are not counted.
  static_assert(kBins == 32 && kWaveHistBytes == 8192, "a lane's word of bin b sits at b << 8 of its base");
  static_assert(kTileBytes % kWaveHistBytes == 0 && (2 * kBufBytes) % kWaveHistBytes == 0,
                "wave histograms start on 8 KB boundaries");
  uint32_t *hwave = reinterpret_cast<uint32_t *>(
      kHistInV ? smem + (wave >> 1) * kBufBytes + kTileBytes + (wave & 1) * kWaveHistBytes
               : smem + 2 * kBufBytes + wave * kWaveHistBytes);
  for (int i = lane; i < 64 * kBins; i += 64) hwave[i] = 0u;
  for (int i = tid; i < (n_kblk + 31) / 32; i += 256) mbits[i] = 0u;
  __syncthreads();
  const float c_h = p.scale * (float)(kBins - 1) * a1;  // z / bw per unit of q.k
  // this lane's words: bin b at hl + (b << 8); the other half of the row's at hl ^ 128
  const uint32_t hl = (uint32_t)(uintptr_t)(lds_char_t *)hwave + (uint32_t)lane * 4u;
  // The anchor sits kAnchorBelow bins below the first maximum, so every bin
  // in the window has a positive index (truncation is the floor there).
  constexpr float kAnchorBelow = 2.f * kBins;
  float m_raw = -INFINITY;  // running row maximum of q.k (both lane halves)
  float anchor = 0.f;       // bin index of the grid origin (an integer)
  float topf = -1e30f;      // bin of the running maximum, from the anchor
  dense_pass([&](int kv0, floatx16_t(&s)[kKt]) {
    float tm = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < kKt; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) tm = fmaxf(tm, s[kt][i]);
    tm = half_max(tm);
    // every live row sees key 0, so its first tile has a finite maximum
    if (kv0 == 0 && tm > -INFINITY) anchor = floorf(tm * c_h) - kAnchorBelow;
    m_raw = fmaxf(m_raw, tm);
    const float ntop = tm > -INFINITY ? floorf(__builtin_fmaf(tm, c_h, -anchor)) : topf;
    // bins (topf, ntop] enter the window: clear their slots (none on the
    // first tile, where every slot is still zero), as many steps as the
    // wave's largest rise (one or two bins once the maximum has settled)
    const float rise = fminf(ntop - topf, (float)kBins);
    if (__builtin_amdgcn_ballot_w64(kv0 > 0 && rise > 0.f) != 0) {
      const int n_clr = rise > 0.f ? (int)rise : 0;
      const int itop = rise > 0.f ? (int)ntop : 0;
      for (int c = 0; __builtin_amdgcn_ballot_w64(c < n_clr) != 0; ++c)
        if (c < n_clr) lds_write_b32(hl + ((uint32_t)((itop - c) & (kBins - 1)) << 8), 0u);
    }
    topf = fmaxf(topf, ntop);
    // t8 = 256 bin, exactly 256 times the unscaled FMA (scaling by a power of
    // two commutes with rounding); counted when bin >= topf - (kBins - 1).
    // Truncating t8 gives 256 floor(t8 / 256) plus 0..255, so masking it
    // with (kBins - 1) << 8 yields the byte offset of the bin's word (mod
    // kBins) directly (t8 > 0 in the window; hl has no bits 8..12).  A score
    // below the window adds 0, so its word may be any of the lane's: the
    // hardware conversion of any t8 serves (it saturates; -inf, for a masked
    // score, gives INT_MIN), written as the instruction itself because the
    // C++ conversion of an out-of-range value is undefined.
    const float lo_t8 = 256.f * (topf - (float)(kBins - 1));
    const float anchor8 = 256.f * anchor;
    const float c_h8 = 256.f * c_h;
#pragma unroll
    for (int kt = 0; kt < kKt; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float t8 = __builtin_fmaf(s[kt][i], c_h8, -anchor8);  // -inf for masked scores
        // every lane adds, 0 for a score below the window (at the window's
        // lowest bin): no branch and exec-mask change per score
        const uint32_t inc = t8 >= lo_t8 ? 1u : 0u;
        uint32_t t8i;
        asm("v_cvt_i32_f32 %0, %1" : "=v"(t8i) : "v"(t8));
        lds_add_u32((t8i & (uint32_t)((kBins - 1) << 8)) | hl, inc);
      }
  });
  const float m = m_raw * p.scale;  // (scale > 0)
  const int n_allowed = p.causal ? qrow + 1 : len;
  // The histogram's root tau_h (both lane halves hold the same row and the
  // same counts, so both compute the same value).  Bin ilo + bb counts at
  // u = (alpha-1) z of its lower edge E_bb = ebase + bb * ebw.  Measured in
  // bins from edge E_k, bin bb > k sits at j = bb - k, so the histogram's
  // mass at E_k is ebw^e G_k with G_k = sum_{bb > k} cnt[bb] j^e: G_k falls
  // with k, G_0 >= 31^e (the top bin holds the maximum) and G_31 = 0, so the
  // root lies in the bin [E_ks, E_ks + ebw) of the largest ks with
  // G_ks >= R = 31^e.  Inside it the mass has no kink: with tau = E_ks + y ebw
  // the root solves H(y) = sum_{bb > ks} cnt[bb] (j - y)^e - R = 0 on [0, 1],
  // in closed form for alpha = 2, by Newton from y = 0 for e >= 1 (H convex
  // and falling: the iterates rise to the root from below, each a lower
  // bound), and by bisection for e < 1.
  const bool counted = topf > -1e29f;  // (rows past the end count nothing)
  const int ilo = counted ? (int)topf - (kBins - 1) : 0;
  float cnt[kBins];
#pragma unroll
  for (int bb = 0; bb < kBins; ++bb) {
    const int w = ((ilo + bb) & (kBins - 1)) * 64;
    cnt[bb] = (float)(hwave[w + lane] + hwave[w + (lane ^ 32)]);
  }
  const float ebw = 1.f / (float)(kBins - 1);  // (alpha-1) bw
  const float ebase = (anchor + (float)ilo) * ebw;
  // d^e and d^(e-1) for d > 0
  auto pw_e = [&](float d) __attribute__((always_inline)) -> float {
    if constexpr (PK == kPowSquare) return d * d;
    else if constexpr (PK == kPowLinear) return d;
    else return __builtin_amdgcn_exp2f(e * __builtin_amdgcn_logf(d));
  };
  float pw[kBins];  // j^e
#pragma unroll
  for (int j = 0; j < kBins; ++j) pw[j] = j == 0 ? 0.f : pw_e((float)j);
  const float R = pw[kBins - 1];
  int ks = 0;
#pragma unroll
  for (int k = 1; k < kBins - 1; ++k) {
    float g = 0.f;
#pragma unroll
    for (int bb = k + 1; bb < kBins; ++bb) g = __builtin_fmaf(cnt[bb], pw[bb - k], g);
    if (g >= R) ks = k;
  }
  float wcnt[kBins], jd[kBins];  // counts of the bins above ks, and their j
#pragma unroll
  for (int bb = 0; bb < kBins; ++bb) {
    wcnt[bb] = bb > ks ? cnt[bb] : 0.f;
    jd[bb] = (float)(bb - ks);
  }
  float y;
  if constexpr (PK == kPowLinear) {
    float s_c = 0.f, s_j = 0.f;
#pragma unroll
    for (int bb = 0; bb < kBins; ++bb) {
      s_c += wcnt[bb];
      s_j = __builtin_fmaf(wcnt[bb], jd[bb], s_j);
    }
    y = (s_j - R) / s_c;
  } else if (e >= 1.f) {
    y = 0.f;
    for (int it = 0; it < 6; ++it) {
      float h = -R, dh = 0.f;
#pragma unroll
      for (int bb = 0; bb < kBins; ++bb) {
        const float d = fmaxf(jd[bb] - y, 1e-30f);
        float de, dm;
        if constexpr (PK == kPowSquare) {
          dm = d;
          de = d * d;
        } else {
          const float l = __builtin_amdgcn_logf(d);
          de = __builtin_amdgcn_exp2f(e * l);
          dm = __builtin_amdgcn_exp2f((e - 1.f) * l);
        }
        h = __builtin_fmaf(wcnt[bb], de, h);
        dh = __builtin_fmaf(wcnt[bb], dm, dh);
      }
      y += h / (e * dh);
    }
  } else {
    float ylo = 0.f, yhi = 1.f;
    for (int it = 0; it < 20; ++it) {
      const float mid = 0.5f * (ylo + yhi);
      float h = -R;
#pragma unroll
      for (int bb = 0; bb < kBins; ++bb) h = __builtin_fmaf(wcnt[bb], pw_e(fmaxf(jd[bb] - mid, 1e-30f)), h);
      if (h >= 0.f)
        ylo = mid;
      else
        yhi = mid;
    }
    y = ylo;
  }
  y = counted ? fminf(fmaxf(y, 0.f), 1.f) : 0.f;
  // less a few ulps, so that rounding leaves it below the histogram's root
  const float tau_h0 = __builtin_fmaf((float)ks + y, ebw, ebase);
  const float tau_h = tau_h0 - 2.5e-7f * fmaxf(1.f, fabsf(tau_h0));
  // ---- pass 2: refinement.  Bracket [blo, bhi] of the true tau: tau_h is
  // below it; counting every score at its bin's upper edge instead would
  // raise every score by at most bw and the root by at most (alpha-1) bw =
  // ebw, so tau_h + ebw is above it (with a little room for fp32 rounding);
  // and at (alpha-1) m - n^(1-alpha) every weight is at most 1/n.
  float blo = tau_h;
  float bhi = fminf(a1 * m - __builtin_amdgcn_exp2f((1.f - p.alpha) *
                                                     __builtin_amdgcn_logf((float)max(n_allowed, 1))),
                    tau_h + ebw * (1.f + 1e-4f) + 1e-6f * fabsf(tau_h));
  if (!(bhi > blo)) bhi = blo + 1e-6f * fmaxf(1.f, fabsf(blo));
  // Starting point: the histogram's root with every score counted at its
  // bin's midpoint, between the lower- and upper-edge placements: that
  // histogram is the lower-edge one moved up by half a bin, so its root is
  // tau_h + ebw / 2 -- close enough that one Halley or Newton step usually
  // finishes the row.
  float t = fminf(fmaxf(tau_h0 + 0.5f * ebw, blo), bhi);
  // regula falsi state (alpha > 2): g at the bracket ends, and which end moved last
  float glo = 0.f, ghi = 0.f;
  int side = 0;
  const float kTol = 4e-6f;  // |sum p - 1| at which a row counts as converged (fp32 sums)
  // Newton (alpha <= 2) and Halley (alpha <= 1.5) converge quadratically and
  // cubically: once |sum p - 1| is below this at the current tau, the step
  // taken from it lands close enough to the root that the row takes it and
  // stops without another pass to confirm it.  Newton from 2e-3 lands within
  // fp32 rounding; Halley from 0.1 within |sum p - 1| ~ 2e-4 at worst (a key
  // entering the support next to the root), which moves O by at most that
  // times max |v - O| (O is divided by sum p), a tenth of O's tolerance.
  const float kStepTol = p.alpha <= 1.5f ? 1e-1f : 2e-3f;
  const float zs = a1 * p.scale;  // (alpha - 1) z = zs * q.k
  bool final_step = false;  // the row took its last step
  const int m_words = (n_kblk + 31) / 32;
  // alpha > 2 (a support of a few keys): the first refinement pass also
  // gathers each row's keys above the bracket's lower end -- every key of the
  // support at the root is one -- and a row with at most kCand of them solves
  // the mass equation on them exactly (bisection in registers to fp32
  // resolution) and stops; near a key entering the support, where the
  // iterative steps crawl, this needs no further pass.  Each lane writes the
  // (alpha-1) z of its own such keys to its histogram words 1, 2, ... (free
  // once the counts are in registers) and counts them in a register; the
  // row's list is its two lane halves' lists together.
  constexpr int kCand = 8;
  const bool gather = PK == kPowGeneral && p.alpha > 2.f;
  uint32_t n_own = 0;  // keys this lane gathered
  for (int r = 0; r < p.n_iter; ++r) {
    const bool first = r == 0;
    // u = (alpha-1) z - t above this: the key is above the bracket's lower end
    // (less a margin for the rounding of u)
    const float c_lo = blo - t - 1e-5f * fmaxf(1.f, fabsf(blo));
    const float t_mask = blo;  // <= every later tau
    // every pass rebuilds the block mask, so the mask of the pass the loop
    // ends after covers the final tau
    for (int w = tid; w < m_words; w += 256) mbits[w] = 0u;
    __syncthreads();
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, shi = 0.f;
    uint32_t n_pos = 0;  // alpha = 1.5: keys with u > 0 (s2), counted as an integer
    // alpha = 2: the u of the nearest key above t and at or below it
    float gap_up = INFINITY, gap_dn = -INFINITY;
    // one tile of the pass; kFirstGt2: the first pass at alpha > 2, which
    // also forms g at the upper bracket end and gathers the keys above the
    // lower one (a separate instantiation keeps those per-score branches out
    // of every other pass)
    auto refine_tile = [&](auto first_gt2_tag, int kv0, floatx16_t(&s)[kKt]) __attribute__((always_inline)) {
      constexpr bool kFirstGt2 = decltype(first_gt2_tag)::value;
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < kKt; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float u = __builtin_fmaf(s[kt][i], zs, -t);
          tmax = fmaxf(tmax, s[kt][i]);
          // s0 = sum u^e, s1 = sum u^(e-1), s2 = sum u^(e-2) over u > 0 (the
          // last two only where the step uses them), without branches
          const float up = fmaxf(u, 0.f);
          const float pos = u > 0.f ? 1.f : 0.f;
          if constexpr (PK == kPowSquare) {
            s0 = __builtin_fmaf(up, up, s0);
            s1 += up;
            n_pos += u > 0.f ? 1u : 0u;
          } else if constexpr (PK == kPowLinear) {
            s0 += up;
            s1 += pos;
            gap_up = fminf(gap_up, u > 0.f ? u : INFINITY);
            gap_dn = fmaxf(gap_dn, u > 0.f ? -INFINITY : u);
          } else if (u > 0.f) {
            const float pu = powpos<PK>(u, e);
            s0 += pu;
            if (p.alpha <= 2.f) {
              const float ru = __builtin_amdgcn_rcpf(u);
              const float r1 = pu * ru;
              s1 += r1;
              if (p.alpha <= 1.5f) s2 += r1 * ru;
            }
          }
          if constexpr (kFirstGt2) {
            shi += powpos<PK>(__builtin_fmaf(s[kt][i], zs, -bhi), e);  // g at the upper end
            if (u > c_lo) {
              if (n_own < (uint32_t)kCand) lds_write_b32(hl + ((n_own + 1u) << 8), __float_as_uint(s[kt][i] * zs));
              ++n_own;
            }
          }
        }
      // mark the 128-key block if some live row's scores clear t_mask
      const bool any = __builtin_amdgcn_ballot_w64(live && zs * tmax > t_mask) != 0;
      if (any && lane == 0)
        lds_or_b32((uint32_t)(uintptr_t)(lds_char_t *)(mbits + kv0 / kListBlock / 32), 1u << ((kv0 / kListBlock) % 32));
    };
    auto plain_pass = [&]() __attribute__((always_inline)) {
      dense_pass([&](int kv0, floatx16_t(&s)[kKt]) { refine_tile(std::false_type{}, kv0, s); });
    };
    if constexpr (PK == kPowGeneral) {
      if (gather && first)
        dense_pass([&](int kv0, floatx16_t(&s)[kKt]) { refine_tile(std::true_type{}, kv0, s); });
      else
        plain_pass();
    } else {
      plain_pass();
    }
    s0 = half_sum(s0);
    s1 = half_sum(s1);
    if constexpr (PK == kPowSquare) s2 = (float)n_pos;
    s2 = half_sum(s2);
    if constexpr (PK == kPowLinear) {
      gap_up = -half_max(-gap_up);
      gap_dn = half_max(gap_dn);
    }
    const float g = s0 - 1.f;
    if (p.alpha > 2.f && first) ghi = half_sum(shi) - 1.f;
    uint32_t n_part = 0;  // keys the other half of the row gathered
    if (gather && first) n_part = (uint32_t)half_sum((float)n_own) - n_own;
    // converged: keep t (the bracket may have closed on it); a row that took
    // its final step keeps the t that step gave; a bracket closed to fp32
    // resolution cannot narrow further
    const bool conv = final_step || fabsf(g) <= kTol || bhi - blo <= 4e-7f * fmaxf(1.f, fabsf(t));
    // close enough for one more Newton / Halley step to land on the root
    const bool last = !conv && p.alpha <= 2.f && fabsf(g) <= kStepTol;
    if (!conv) {
      if (g > 0.f) {
        blo = t;
        glo = g;
        if (side == 1) ghi *= 0.5f;  // Illinois: the other end stayed twice
        side = 1;
      } else {
        bhi = t;
        ghi = g;
        if (side == -1) glo *= 0.5f;
        side = -1;
      }
      float t_new;
      if (p.alpha <= 1.5f) {  // Halley
        const float g1 = -e * s1, g2 = e * (e - 1.f) * s2;
        t_new = t - 2.f * g * g1 / (2.f * g1 * g1 - g * g2);
      } else if (p.alpha <= 2.f) {  // Newton
        t_new = t - g / (-e * s1);
      } else {  // secant through the bracket ends (regula falsi)
        t_new = ghi < glo ? blo - glo * (bhi - blo) / (ghi - glo) : 0.5f * (blo + bhi);
      }
      const bool inside = t_new >= blo && t_new <= bhi;
      // alpha = 2: the mass is linear in tau while no key enters or leaves the
      // support, so a Newton step that stays between the nearest keys on
      // either side of t lands on the root (to rounding) whatever g was
      bool exact = false;
      if constexpr (PK == kPowLinear) exact = t_new - t < gap_up && t_new - t > gap_dn;
      t = inside ? t_new : 0.5f * (blo + bhi);  // bisection fallback (then not a last step)
      final_step = (last || exact) && inside;
      if (gather && first) {
        const uint32_t n_c = n_own + n_part;
        if (n_c <= (uint32_t)kCand) {  // the exact root on the gathered keys
          float cv[kCand];
#pragma unroll
          for (int i = 0; i < kCand; ++i) {
            const uint32_t j = (uint32_t)i < n_own ? (uint32_t)i : (uint32_t)i - n_own;
            const int src = (uint32_t)i < n_own ? lane : (lane ^ 32);
            cv[i] = (uint32_t)i < n_c ? __uint_as_float(hwave[(int)(j + 1u) * 64 + src]) : -INFINITY;
          }
          float xlo = blo, xhi = bhi;
          for (int it = 0; it < 24; ++it) {
            const float mid = 0.5f * (xlo + xhi);
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < kCand; ++i) sum += powpos<PK>(cv[i] - mid, e);
            if (sum >= 1.f)
              xlo = mid;
            else
              xhi = mid;
          }
          t = 0.5f * (xlo + xhi);
          final_step = true;
        }
      }
    }
    // the workgroup stops once every live row has converged or taken its last step
    const bool wave_done = __builtin_amdgcn_ballot_w64(live && !conv && !final_step) == 0;
    if (lane == 0) done_flag[wave] = wave_done ? 1u : 0u;
    __syncthreads();
    const bool all_done = done_flag[0] & done_flag[1] & done_flag[2] & done_flag[3];
    if (all_done) break;
    // (the flags are rewritten only after the next pass's barriers)
  }
  __syncthreads();  // the mask is complete

  // ---- pass 3: output over the marked blocks
  floatx16_t oacc[kDt];
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float l = 0.f;
  int n_blk = 0;
  for (int w = 0; w < m_words; ++w) n_blk += __builtin_popcount(mbits[w]);
  const int n_out = kTpb * n_blk;
  int c_w = -1;
  uint32_t c_bits = 0;
  int c_blk = 0;
  auto out_kv = [&](int it) -> int {  // in order
    if (it % kTpb == 0) {
      while (c_bits == 0) c_bits = mbits[++c_w];
      c_blk = 32 * c_w + __builtin_ctz(c_bits);
      c_bits &= c_bits - 1u;
    }
    return c_blk * kListBlock + (it % kTpb) * kBN;
  };
  uint32_t vlds[kDt];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_char_t *)smem;
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt)
    vlds[dt] = smem_lds + (uint32_t)L::vv(4 * hi + (j16 >> 2), 2 * dt + (l32 >> 4), (j16 & 3) * 8);
  int kv_cur = n_out > 0 ? out_kv(0) : 0;
  if (n_out > 0) issue(0, kv_cur, true);
  for (int it = 0; it < n_out; ++it) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    int kv_nxt = 0;
    if (it + 1 < n_out) {
      kv_nxt = out_kv(it + 1);
      issue((it + 1) & 1, kv_nxt, true);
    }
    const int kv0 = kv_cur;
    kv_cur = kv_nxt;
    const int boff = (it & 1) * kBufBytes;
    floatx16_t s[kKt];
    scores(boff, kv0, s);
    bf16x8_t pb[kKt][2];
#pragma unroll
    for (int kt = 0; kt < kKt; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = powpos<PK>(__builtin_fmaf(s[kt][i], zs, -t), e);
        l += pv;
        pb[kt][i >> 3][i & 7] = (__bf16)pv;
      }
    {
      // O^T += V^T P^T: V^T operands by transpose reads kRing MFMAs ahead,
      // consecutive MFMAs alternating between the kDt accumulators (step i:
      // dt = i % kDt, (kt, c) = i / kDt)
      uint32_t vb[kDt];
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) vb[dt] = vlds[dt] + boff + kTileBytes;
      constexpr int kRing = 4;
      constexpr int kSteps = kDt * kKt * 2;
      bf16x8_t ring[kRing];
      static_for<kRing>([&](auto I) {
        constexpr int i = decltype(I)::value;
        ring[i] = tr_pair<tr_off<L, kDt>(i), 8 * kRowBytes>(vb[i % kDt]);
      });
      static_for<kSteps>([&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr int dt = i % kDt, kc = i / kDt;
        // LDS reads complete in order: step i's are done once at most the
        // reads issued after them are outstanding
        lgkm_wait<2 * (kSteps - 1 - i < kRing - 1 ? kSteps - 1 - i : kRing - 1)>(ring[i % kRing]);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], pb[kc >> 1][kc & 1], oacc[dt], 0, 0, 0);
        if constexpr (i + kRing < kSteps)
          ring[i % kRing] = tr_pair<tr_off<L, kDt>(i + kRing), 8 * kRowBytes>(vb[(i + kRing) % kDt]);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  const float l_tot = half_sum(l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // ---- epilogue: O (bf16), tau, tau_h, the mask row
  if (live) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int dcol = dt * 32 + (i >> 2) * 8 + hi * 4 + (i & 3);
        og[(int64_t)qrow * p.o_ss + dcol] = __builtin_bit_cast(uint16_t, (__bf16)(oacc[dt][i] * inv));
      }
    if (hi == 0) {
      const int64_t idx = ((int64_t)b * p.hq + h) * p.seqlen + qrow;
      if (p.tau) p.tau[idx] = t;
      if (p.tau_init) p.tau_init[idx] = tau_h;
    }
  }
  if (p.mask) {
    uint32_t *mrow = p.mask + (((int64_t)b * p.hq + h) * p.n_tiles + tile) * p.mask_words;
    for (int w = tid; w < p.mask_words; w += 256) mrow[w] = w < m_words ? mbits[w] : 0u;
  }
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
bool stride_ok(int64_t s) { return ((s * 2) % 16) == 0; }

}  // namespace

extern "C" int attn_entmax_fwd_validate(const attn_tensor_t *q, const attn_tensor_t *k,
                                        const attn_tensor_t *v, int causal, float scale,
                                        float alpha, int n_iter, const attn_tensor_t *out,
                                        int mask_words) {
  const int st = attn_fwd_validate(q, k, v, nullptr, causal, scale, nullptr, out);
  if (st != ATTN_OK) return st;
  if (!isfinite(alpha) || !(alpha > 1.f) || n_iter < 1 || n_iter > 32) return ATTN_ERR_INVALID_ARG;
  // Above alpha = 3 the weights u^(1/(alpha-1)) rise so steeply from the
  // support edge that fp32 scores cannot reproduce exact weights to the
  // forward's tolerances (a key 1e-6 above the edge already weighs 0.03 at
  // alpha = 5); below 1.05 the window 1/(alpha-1) outgrows fp32 range use.
  if (alpha > 3.f || alpha < 1.05f) return ATTN_ERR_UNSUPPORTED;
  const int64_t n_blk = (q->seqlen + kListBlock - 1) / kListBlock;
  if (n_blk > kMaxKBlocks) return ATTN_ERR_UNSUPPORTED;
  if (mask_words < 0) return ATTN_ERR_INVALID_ARG;
  if (mask_words > 0 && (int64_t)mask_words * 32 < n_blk) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

extern "C" int attn_entmax_fwd(const attn_tensor_t *q, const attn_tensor_t *k,
                               const attn_tensor_t *v, int causal, float scale, float alpha,
                               int n_iter, attn_tensor_t *out, float *tau, uint32_t *block_mask,
                               int mask_words, float *tau_init, void *stream) {
  const int st = attn_entmax_fwd_validate(q, k, v, causal, scale, alpha, n_iter, out,
                                          block_mask ? mask_words : 0);
  if (st != ATTN_OK) return st;
  if (q->batch == 0 || q->seqlen == 0) return ATTN_OK;
  EntParams p;
  p.q = static_cast<const uint16_t *>(q->data);
  p.k = static_cast<const uint16_t *>(k->data);
  p.v = static_cast<const uint16_t *>(v->data);
  p.o = static_cast<uint16_t *>(out->data);
  p.tau = tau;
  p.tau_init = tau_init;
  p.mask = block_mask;
  p.mask_words = mask_words;
  p.q_sb = q->stride_batch; p.q_ss = q->stride_seq; p.q_sh = q->stride_head;
  p.k_sb = k->stride_batch; p.k_ss = k->stride_seq; p.k_sh = k->stride_head;
  p.v_sb = v->stride_batch; p.v_ss = v->stride_seq; p.v_sh = v->stride_head;
  p.o_sb = out->stride_batch; p.o_ss = out->stride_seq; p.o_sh = out->stride_head;
  p.batch = q->batch;
  p.seqlen = q->seqlen;
  p.hq = q->heads;
  p.group = q->heads / k->heads;
  p.n_tiles = (q->seqlen + 127) / 128;
  p.n_iter = n_iter;
  p.causal = causal;
  p.scale = scale;
  p.alpha = alpha;
  const int64_t grid = (int64_t)p.n_tiles * p.batch * p.hq;
  void *args[] = {&p};
  // integer exponents (alpha = 2: e = 1; alpha = 1.5: e = 2) take the
  // instantiation without transcendentals
  const int pk = alpha == 2.f ? kPowLinear : (alpha == 1.5f ? kPowSquare : kPowGeneral);
  const void *fns[3][3] = {
      {reinterpret_cast<const void *>(&attn_entmax_kernel<64, kPowGeneral>),
       reinterpret_cast<const void *>(&attn_entmax_kernel<64, kPowLinear>),
       reinterpret_cast<const void *>(&attn_entmax_kernel<64, kPowSquare>)},
      {reinterpret_cast<const void *>(&attn_entmax_kernel<128, kPowGeneral>),
       reinterpret_cast<const void *>(&attn_entmax_kernel<128, kPowLinear>),
       reinterpret_cast<const void *>(&attn_entmax_kernel<128, kPowSquare>)},
      {reinterpret_cast<const void *>(&attn_entmax_kernel<256, kPowGeneral>),
       reinterpret_cast<const void *>(&attn_entmax_kernel<256, kPowLinear>),
       reinterpret_cast<const void *>(&attn_entmax_kernel<256, kPowSquare>)}};
  const void *fn = fns[q->head_dim == 64 ? 0 : (q->head_dim == 128 ? 1 : 2)][pk];
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
