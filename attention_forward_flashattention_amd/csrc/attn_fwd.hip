// attn_fwd.hip — fused softmax-attention forward for AMD Instinct MI355X (gfx950).
//
// One workgroup computes a tile of query rows of one (sequence, query head):
// for dense and packed problems 256 rows in eight wave64s (head_dim 128), 384
// rows in twelve (head_dim 64) or 128 rows in four (head_dim 256).  The
// block-list, block-mask and ordered-skipping kernels take one 128-row query
// block of the list or mask, for two query heads of a GQA group in eight
// wave64s (or for one head in four).  Each wave owns 32 rows and keeps them in
// registers for the whole kernel.  KV tiles of BN keys (64; 32 at head_dim
// 256) are streamed into a ring of LDS slots with direct global-to-LDS loads;
// for each tile a wave computes the transposed
// score tile S^T = K Q^T with 32x32x16 bf16 MFMAs, so that every lane holds
// the scores of ONE query row (the softmax row statistics then need one
// exchange between the two lane halves instead of a 32-lane reduction), runs
// the online softmax in base 2 with scale*log2(e) folded into one FMA, and
// accumulates O^T = V^T P^T with the same MFMA, P staying in registers.  V^T
// operands come straight from the row-major V tile with the gfx950 LDS
// transpose read (ds_read_b64_tr_b16).
//
// The computation is the softmax attention that FlashAttention-style kernels
// evaluate tile by tile in on-chip memory (AdaSplash-2 explainer, technical
// summary section 1); block skipping follows the ordered per-query-block KV
// list of the CoSA explainer (lay summary): unlisted blocks are never loaded,
// and in the ordered-skipping mode the walk along the list also stops once the
// blocks still listed can add little to what the first ones gathered.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <utility>

#include "attn_common.h"
#include "attn_fwd.h"

namespace {

using namespace attn_detail;

// A tile's P is accepted against the running max while every row sum of the
// tile stays at or below this (so every P is at most 2^12).
constexpr float kFastSum = 4096.f;

struct Params {
  const uint16_t *q, *k, *v;
  uint16_t *o;
  float *lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  const int32_t *cu;       // packed sequences, or null
  const int32_t *row_ptr;  // block list, or null
  const int32_t *col_idx;
  const uint32_t *mask;    // bit-packed block mask, or null
  int64_t mask_ss, mask_sh; // words between masks of consecutive sequences / kv heads
  int mask_words;          // words per query-block row of a mask
  float osk_tau;           // ordered skipping: stop when (entries left) x every row's newest-entry mass <= tau x its mass
  int osk_min_visit;       // ... but never before this many entries
  int32_t *visited;        // ordered skipping: entries visited per (query head, query block), or null
  int batch, seqlen, hq, group;
  int n_tiles;   // query tiles per (sequence, head) = ceil(seqlen / BM)
  int n_units;   // batch * (hq / query heads per workgroup)
  int unit_group;  // units per KV head (group / query heads per workgroup)
  int group_major; // 1: each XCD takes its groups one after another; 2: the chip takes them one after another (see decode_tile)
  int xcd_remap; // 1 when n_units % (8 * unit_group) == 0 (whole GQA groups dealt over the 8 XCDs)
  float c;       // scale * log2(e)
};

// Kernel configuration.  NW wave64s per workgroup, each owning 32 query rows
// (BM = 32 * NW rows per workgroup); BN keys per KV tile (64, or 32 at head_dim
// 256 to bound registers and LDS).  Dense and packed problems use 8 waves at
// head_dim 128 (two per SIMD, 256-row tiles: every K/V tile staged in LDS
// serves 256 query rows) and 12 at head_dim 64 (three per SIMD: the
// pipelined loop needs under 168 VGPRs there, so a third wave fits and hides
// more of each wave's serial barrier and load-issue time); the block-list,
// block-mask and ordered-skipping kernels use 8 waves for one 128-row query
// block of two query heads of a GQA group, or 4 for one head.
template <int D_, int NW_>
struct Config {
  static constexpr int D = D_;
  static constexpr int NW = NW_;
  static constexpr int kThreads = 64 * NW;
  static constexpr int kBM = 32 * NW;
  static constexpr int kBN = D == 256 ? 32 : 64;
  static constexpr int kTileBytes = kBN * D * 2;
  // waves that load K/V tiles (the first kLoadWaves) and their wave-wide 16 B
  // loads per tile each
  static constexpr int kLoadWaves = NW < 8 ? NW : 8;
  static constexpr int kLoads = kTileBytes / 1024 / kLoadWaves;
  static_assert(kLoads * 1024 * kLoadWaves == kTileBytes, "tile must split evenly over the loading waves");
  static constexpr int kMinBlocks = (NW == 4 && D <= 128) ? 2 : 1;  // 2 waves per SIMD
};

// P = 2^(c s - m) for one tile of scores, rounded to bf16 in the MFMA
// operand layout; returns this lane's sum of the unrounded P.
template <int kKt>
__device__ __forceinline__ float exp_tile(const floatx16_t (&s)[kKt], float c, float m,
                                          bf16x8_t (&pb)[kKt][2]) {
  float rs = 0.f;
#pragma unroll
  for (int kt = 0; kt < kKt; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], c, -m));
      rs += pv;
      pb[kt][i >> 3][i & 7] = (__bf16)pv;
    }
  return rs;
}

// Decode the workgroup id into (query tile, unit); a unit is one sequence and
// one (or, for the paired block-sparse kernels, two) query heads.  Workgroups
// are dealt round-robin over the 8 XCDs (each with its own L2).  When the
// units split evenly, the `unit_group` units that share one KV head stay
// together and those groups are dealt round-robin over the XCDs, so every XCD
// gets the same mix of sequences (packed batches stay balanced) and the heads
// that read the same K/V share one L2.  Within an XCD, when every CU gets many
// workgroups, the groups follow one another (all tiles of a group before the
// next), so the workgroups in flight on an XCD read the same K/V prefix and it
// stays in the XCD's L2 (packed D=256: +9%); with few workgroups per CU the
// tiles go tile by tile over all of the XCD's units, which balances the CUs
// (dense MHA S=2048: the group order there is 28% slower).  The block-list
// and block-mask kernels with many workgroups per CU take a third order: the
// whole chip works on one KV head's group at a time (the group's tiles,
// heaviest first, dealt round-robin over the XCDs, the units of one query
// block on one XCD one after the other).  Their listed blocks lie anywhere
// below the diagonal, so little of them is reused from an XCD's L2; with one
// KV head in flight the K/V that the chip reads at a time is that head's
// (64 MB at a 128K context), which the 256 MB Infinity Cache holds, where
// eight heads in flight (one per XCD) would not fit (128K list and mask
// workloads: 2-3% faster; ordered skipping keeps the per-XCD order, 1%
// better there).  Causal and block-list tiles are issued heaviest first.
__device__ __forceinline__ void decode_tile(const Params &p, bool heavy_first, int &tile,
                                            int &unit) {
  const int w = blockIdx.x;
  int rank;
  if (p.xcd_remap) {
    const int upx = p.n_units >> 3;  // units per XCD
    const int xcd = w & 7;
    const int local = w >> 3;
    if (p.group_major == 2) {
      // chip-wide: slot = (group, rank) in order; XCD = slot mod 8
      const int ug = p.unit_group;
      const int slot = (local / ug) * 8 + xcd;
      const int g = slot / p.n_tiles;
      rank = slot % p.n_tiles;
      unit = g * ug + local % ug;
    } else if (p.group_major) {
      // all tiles of one KV head's units (heaviest first), then the next
      const int per_group = p.unit_group * p.n_tiles;
      const int gi = local / per_group;
      const int r = local % per_group;
      rank = r / p.unit_group;
      unit = (gi * 8 + xcd) * p.unit_group + r % p.unit_group;
    } else {
      // tile by tile (heaviest first) over all of this XCD's units
      rank = local / upx;
      const int lu = local % upx;  // unit slot within this XCD
      unit = ((lu / p.unit_group) * 8 + xcd) * p.unit_group + lu % p.unit_group;
    }
  } else {
    rank = w / p.n_units;
    unit = w % p.n_units;
  }
  tile = heavy_first ? p.n_tiles - 1 - rank : rank;
}

// A wave-uniform read of the block list or the block mask, through the
// constant address space: neither is written while a kernel runs, so the
// compiler may use a scalar load.  (A plain load in the main loop, after
// direct-to-LDS loads that it cannot tell from stores, becomes a vector load
// that the wave waits for at once: a full memory latency per list entry.)
template <class T>
__device__ __forceinline__ T ld_uniform(const T *base, int64_t i) {
  return ((const __attribute__((address_space(4))) T *)base)[i];
}

// Direct global -> LDS loads of the rows of one K or V tile.  Each wave-wide
// load writes 64 consecutive 16 B LDS slots; each lane fetches the global
// chunk that the swizzled layout places in its slot.  The per-lane part of the
// global offset (off, in bytes: row lrow0 + n * (64 / kChunks) of the tile for
// load n) is fixed for the whole kernel and fits 32 bits (the host bounds the
// row stride); only the tile's start address t0, uniform over the wave,
// changes, so each load takes one 32-bit register offset from a scalar base.
// In a tile that runs past the end of the sequence the missing rows re-read
// the last row (finite data; those keys are masked).
template <class C>
__device__ __forceinline__ void issue_rows(char *dst, const char *t0, const uint32_t *off, int lrow0,
                                           uint32_t ss_bytes, int rows_left) {
  constexpr int kLoads = C::kLoads;
  constexpr int kRowStep = 64 / (C::D / 8);  // tile rows between a lane's consecutive loads
  // (the empty asm keeps each offset a 32-bit value at its load: widened
  // outside the loop it would take a register pair and the 64-bit address form)
  if (rows_left >= C::kBN) {
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      uint32_t o = off[n];
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(t0 + o, (lds_void_t *)(dst + n * 1024), 16, 0, 0);
    }
  } else {
    // Rows from r_last + 1 on re-read row r_last (the sequence's last row,
    // relative to t0).  A tile that starts at or past the end (a sub-tile of a
    // ragged last block of a block list or mask: rows_left <= 0) has r_last < 0;
    // its base then moves back to that row, so that every lane steps back by
    // at most its own row and the unsigned offset stays >= 0.
    const int r_last = rows_left - 1;
    const int base_row = min(r_last, 0);
    const char *const tb = t0 + (int64_t)base_row * ss_bytes;
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      const int lrow = lrow0 + n * kRowStep;
      const uint32_t back = (uint32_t)(max(lrow - r_last, 0) + base_row);  // 0 <= back <= lrow
      uint32_t o = off[n] - back * ss_bytes;
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(tb + o, (lds_void_t *)(dst + n * 1024), 16, 0, 0);
    }
  }
}

// The 32 Q rows of one wave (from row `row0`, rows from `len` on re-reading
// row len - 1) into LDS at `dst` in the K tiles' swizzled layout, with
// whole-row 16 B loads.
template <int kRowBytes, int kChunks, int kRowsPerWin>
__device__ __forceinline__ void stage_q_rows(char *dst, const uint16_t *qg, int64_t q_ss, int row0, int len,
                                             int lane) {
  constexpr int kQLoads = 32 * kRowBytes / 1024;
  // (the empty asm keeps the compiler from sharing these lane offsets with the
  // epilogue's similar ones, which would keep them live through the main loop)
  asm volatile("" : "+v"(lane));
#pragma unroll
  for (int n = 0; n < kQLoads; ++n) {
    const int slot = n * 64 + lane;
    const int r = slot / kChunks, pc = slot % kChunks;
    const int64_t row = row0 + r < len ? row0 + r : len - 1;
    const int swz = (r / kRowsPerWin) % kChunks;  // the K tiles' chunk swizzle
    __builtin_amdgcn_global_load_lds(qg + row * q_ss + (pc ^ swz) * 8, (lds_void_t *)(dst + n * 1024), 16, 0, 0);
  }
}

// One KV tile (K then V) into one LDS buffer.
template <class C>
__device__ __forceinline__ void issue_tile(char *kb, char *vb, const char *kt0, const char *vt0,
                                           const uint32_t *koff, const uint32_t *voff, int lrow0,
                                           uint32_t k_ssb, uint32_t v_ssb, int rows_left) {
  issue_rows<C>(kb, kt0, koff, lrow0, k_ssb, rows_left);
  issue_rows<C>(vb, vt0, voff, lrow0, v_ssb, rows_left);
}

// Byte distance between the V operand offsets of output tile dt and of tile
// dt % kVRegs (the V pair swizzle repeats every kVRegs tiles of 32 columns).
template <int kVRegs>
__host__ __device__ constexpr int v_imm(int dt) { return (dt / kVRegs) * kVRegs * 64; }

// Operand steps of one MFMA phase of the pipelined dense loop: scores of one
// tile and PV of the previous one interleaved (kBoth), or one of them alone.
// Step t is a score MFMA (kind 0, one 16 B K read) or a PV MFMA (kind 1, two
// transpose reads of V), with index x among the steps of its kind.
enum { kBoth = 0, kOnlyS = 1, kOnlyPV = 2 };
__host__ __device__ constexpr int step_kind(int w, int t) { return w == kBoth ? (t & 1) : (w == kOnlyS ? 0 : 1); }
__host__ __device__ constexpr int step_idx(int w, int t) { return w == kBoth ? (t >> 1) : t; }
__host__ __device__ constexpr int step_reads(int w, int t) { return step_kind(w, t) == 0 ? 1 : 2; }
// LDS reads still allowed in flight when step i needs its operand: those of
// the steps after it that a ring of r operands has already issued.
__host__ __device__ constexpr int step_wait(int w, int n, int r, int i) {
  int c = 0;
  for (int t = i + 1; t < n && t < i + r; ++t) c += step_reads(w, t);
  return c;
}

template <class C, bool CAUSAL, int MODE>
__global__ __launch_bounds__(C::kThreads, C::kMinBlocks) void attn_fwd_kernel(Params p) {
  constexpr int D = C::D;
  constexpr bool LIST = MODE != kDense;  // block-sparse: one 128-row query block per workgroup
  constexpr bool OSK = MODE == kOsk;     // block list with ordered skipping
  using L = Lds<D>;
  constexpr int kBM = C::kBM;
  constexpr int kBN = C::kBN;
  constexpr int kDc = D / 16;   // MFMA k-steps over the head dimension
  constexpr int kDt = D / 32;   // 32-row output tiles over the head dimension
  constexpr int kKt = kBN / 32; // 32-key score tiles per KV tile
  constexpr int kTileBytes = C::kTileBytes;
  constexpr int kBufBytes = 2 * kTileBytes;  // one K tile then one V tile
  // With one workgroup per CU the O staging area of the epilogue has LDS of its
  // own, so a wave can write out its rows while others still read K/V.
  constexpr bool kOwnStage = C::kMinBlocks == 1;
  constexpr int kStageBytes = C::NW * 32 * D * 2;
  constexpr int kFlagBytes = OSK ? 4 * C::NW : 0;  // one stop flag per wave
  // Problems with two waves per SIMD from one workgroup (dense, or the
  // paired block-list, block-mask and ordered-skipping kernels) run the
  // software-pipelined loop below, and so does head_dim 256 (one wave per
  // SIMD, in its solo form); the other kernels (block lists of unpaired heads,
  // ordered skipping at head_dim 256 or unpaired) the plain one.
  constexpr bool kSolo = !OSK && C::NW == 4 && D == 256;
  constexpr bool kPipe = C::NW >= 8 || kSolo;
  // K/V tiles in LDS.  Pipelined loop: a ring of kStages slots, all K tiles
  // first (slot b at b * kTileBytes), then all V tiles (slot b at
  // kStages * kTileBytes + b * kTileBytes), so that every operand read's
  // immediate offset stays below 64 KiB.  Three slots (loads issued two
  // tiles ahead) at head_dim 256, whose 32-key tiles leave one iteration too
  // little time for a load to land (+7% there); two elsewhere (a third slot
  // gained nothing at 64 and 128, and 64-key tiles of block-sparse lists
  // lose to random addresses no matter how early they are issued).  Plain
  // loop: two buffers of [K tile, V tile].
  constexpr int kStages = (kPipe && D == 256) ? 3 : 2;
  constexpr int kKVBytes = kStages * kBufBytes;
  __shared__ __attribute__((aligned(1024))) char smem[kKVBytes + (kOwnStage ? kStageBytes : 0) + kFlagBytes];
  uint32_t *osk_flag = reinterpret_cast<uint32_t *>(smem + kKVBytes + (kOwnStage ? kStageBytes : 0));
  auto kslot = [](int b) { return b * kTileBytes; };
  auto vslot = [](int b) { return kStages * kTileBytes + b * kTileBytes; };

  // Query heads per workgroup: the pipelined block-list, block-mask and
  // ordered-skipping kernels take two query heads of one GQA group, 128 rows
  // (one query block) each; the two share the KV head and the block set, so
  // every K/V tile staged in LDS serves both, as a 256-row dense tile does.
  constexpr int kHpw = (LIST && C::NW == 8) ? 2 : 1;
  constexpr int kWph = C::NW / kHpw;  // waves per query head
  constexpr int kRows = kBM / kHpw;   // query rows per workgroup and head
  static_assert(!LIST || kRows == kListBlock, "one query block per workgroup and head");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;  // lane half
  const int j16 = lane & 15;

  int tile, unit;
  decode_tile(p, CAUSAL || LIST, tile, unit);
  const int n_hu = p.hq / kHpw;                       // units per sequence
  const int b = unit / n_hu;
  const int h = (unit % n_hu) * kHpw + wave / kWph;   // this wave's query head
  const int kvh = ((unit % n_hu) * kHpw) / p.group;   // the workgroup's KV head

  int64_t tok0 = 0;
  int len = p.seqlen;
  if (p.cu) {
    tok0 = p.cu[b];
    len = p.cu[b + 1] - p.cu[b];
  }
  const int q0 = tile * kRows;
  if (q0 >= len) return;
  const int w_row0 = q0 + (wave % kWph) * 32;  // this wave's first query row

  const uint16_t *qg = p.q + (p.cu ? tok0 * p.q_ss : (int64_t)b * p.q_sb) + (int64_t)h * p.q_sh;
  const uint16_t *kg = p.k + (p.cu ? tok0 * p.k_ss : (int64_t)b * p.k_sb) + (int64_t)kvh * p.k_sh;
  const uint16_t *vg = p.v + (p.cu ? tok0 * p.v_ss : (int64_t)b * p.v_sb) + (int64_t)kvh * p.v_sh;
  uint16_t *og = p.o + (p.cu ? tok0 * p.o_ss : (int64_t)b * p.o_sb) + (int64_t)h * p.o_sh;

  // ---- KV iteration space
  constexpr int kSub = kListBlock / kBN;  // KV tiles per 128-key block
  // (the stop flags of an entry are written after its last tile and read after
  // the barrier that starts the next entry: two tiles per entry keep a write
  // from racing a read of the previous flags)
  static_assert(!OSK || kSub >= 2, "ordered skipping needs two or more tiles per list entry");
  int n_iter;
  int e0 = 0, n_ent = 0;
  // this query block's list entries (col_idx + e0): one pointer kept instead of
  // the list base and e0, which left the walk reloading spilled SGPRs from
  // VGPR lanes at every entry (128K list: 2.8% faster)
  const int32_t *crow = p.col_idx;
  const int n_kvblk = (len + kListBlock - 1) / kListBlock;
  // block mask: this query block's row of the (sequence, kv head) mask; under
  // causal masking only blocks up to the query block count
  const uint32_t *mrow = nullptr;
  const int m_lim = CAUSAL ? min(n_kvblk, tile + 1) : n_kvblk;
  const int m_words = (m_lim + 31) >> 5;
  auto m_valid = [&](int w) -> uint32_t {  // bits of word w below m_lim
    const int left = m_lim - 32 * w;
    return left >= 32 ? 0xffffffffu : (left <= 0 ? 0u : ((1u << left) - 1u));
  };
  if (MODE == kList || MODE == kOsk) {
    e0 = p.row_ptr[tile];
    n_ent = p.row_ptr[tile + 1] - e0;
    crow = p.col_idx + e0;
    n_iter = n_ent * kSub;
  } else if (MODE == kMask) {
    mrow = p.mask + b * p.mask_ss + kvh * p.mask_sh + (int64_t)tile * p.mask_words;
    // set bits below m_lim, one word per lane, summed over the wave
    int n_blk = 0;
    for (int w0 = 0; w0 < m_words; w0 += 64) {
      const int w = w0 + lane;
      n_blk += wave_sum(w < m_words ? __builtin_popcount(mrow[w] & m_valid(w)) : 0);
    }
    n_iter = __builtin_amdgcn_readfirstlane(n_blk) * kSub;
  } else {
    const int kv_end = CAUSAL ? min(len, q0 + kRows) : len;
    n_iter = (kv_end + kBN - 1) / kBN;
  }
  // kv start of iteration `it` (called for it = 0, 1, 2, ... in order), or -1
  // to skip it (block-list ids out of range or, under causal masking, wholly
  // above this query tile).  The mask is walked set bit by set bit: lowest
  // bit first, words in order.
  int m_w = -1;        // mask word being walked
  uint32_t m_bits = 0; // its set bits not yet visited
  int m_blk = 0;       // block of the current iteration
  auto kv_start = [&](int it) -> int {
    if (MODE == kDense) return it * kBN;
    if (MODE == kMask) {
      if (it % kSub == 0) {
        while (m_bits == 0) {
          if (++m_w >= m_words) return -1;
          m_bits = ld_uniform(mrow, m_w) & m_valid(m_w);
        }
        m_blk = 32 * m_w + __builtin_ctz(m_bits);
        m_bits &= m_bits - 1u;
      }
      return m_blk * kListBlock + (it % kSub) * kBN;
    }
    const int cb = ld_uniform(crow, it / kSub);
    if (cb < 0 || cb >= n_kvblk) return -1;
    if (CAUSAL && cb * kListBlock > q0 + kRows - 1) return -1;
    return cb * kListBlock + (it % kSub) * kBN;
  };

  // Direct global -> LDS loads of one KV tile into buffer `buf`.  Each wave-wide
  // load writes 64 consecutive 16 B LDS slots; each lane fetches the global
  // chunk that the swizzled layout places in its slot.  The per-lane part of
  // the global offset is fixed for the whole kernel; only the tile's start row
  // changes.  In a tile that runs past the end of the sequence the missing
  // rows re-read the last row (finite data; those keys are masked).
  constexpr int kLoads = C::kLoads;
  static_assert(64 % L::kChunks == 0, "a wave-wide load covers whole rows");
  uint32_t koff[kLoads], voff[kLoads];  // byte offsets within a tile's rows
  // waves past the loading ones issue no loads (their offsets are unused)
  const bool loader = C::NW <= C::kLoadWaves || wave < C::kLoadWaves;
  const int lwave = wave % C::kLoadWaves;
  const int slot_byte0 = lwave * kLoads * 1024;  // this wave's first LDS slot in a tile
  const int lrow0 = (lwave * kLoads * 64 + lane) / L::kChunks;  // row of this lane's first load
  const uint32_t k_ssb = (uint32_t)p.k_ss * 2u, v_ssb = (uint32_t)p.v_ss * 2u;  // row strides in bytes
#pragma unroll
  for (int n = 0; n < kLoads; ++n) {
    const int slot = (lwave * kLoads + n) * 64 + lane;
    const int r = slot / L::kChunks, pc = slot % L::kChunks;
    koff[n] = (uint32_t)r * k_ssb + (uint32_t)(pc ^ L::kswz(r)) * 16u;
    voff[n] = (uint32_t)r * v_ssb + (uint32_t)L::v_logical_chunk(r, pc) * 16u;
  }
  // tile base addresses (bytes), uniform over the workgroup
  const char *const kgb = reinterpret_cast<const char *>(kg);
  const char *const vgb = reinterpret_cast<const char *>(vg);
  auto kt_at = [&](int pos) { return kgb + (int64_t)pos * k_ssb; };
  auto vt_at = [&](int pos) { return vgb + (int64_t)pos * v_ssb; };

  floatx16_t oacc[kDt];
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  // Running max of c*s for this lane's row (c = scale*log2 e).  It is raised
  // lazily (see the softmax step below), so most tiles neither take the
  // tile's max nor rescale O.
  float m_run = -INFINITY;
  float l_run = 0.f;  // running sum over this lane's half of the keys
  float d_run = 0.f;  // ordered skipping: the current list entry's part of l_run

  const int qrow = w_row0 + l32;  // this lane's query row (sequence position)
  const int wq_last = w_row0 + 31;

  int kv_cur = -1;  // plain loop: first key of the tile in flight

  // ---- tile walk of the pipelined loop.  Each tile has a load position (its
  // first key) and a mask position: the same, or far past every key (the
  // whole tile masked) for a list entry that names no block of the sequence,
  // which is loaded from block 0.  Dense: tile t starts at key t*kBN.  Block
  // list and mask: tile t is sub-tile t % kSub of the (t / kSub)-th visited
  // block, visited in list order (mask: set bits, lowest first).  The next
  // list entry (mask word) is read one entry ahead, so its scalar load has a
  // whole entry's tiles to land before it is needed.
  constexpr int kFarKey = 1 << 30;
  int w_t = 0;          // dense: next tile
  int w_sub = kSub;     // sub-tile of the current entry (kSub: go to the next entry)
  int w_ent = -1;       // list: current entry
  int w_blk = 0;        // current block
  bool w_ok = true;     // it lies in the sequence
  int w_raw = (kPipe && (MODE == kList || OSK) && n_ent > 0) ? ld_uniform(crow, 0) : 0;  // id of entry w_ent + 1
  int mw_w = -1;        // mask: word being walked
  uint32_t mw_bits = 0u;  // its set bits not yet visited
  uint32_t mw_pf = (kPipe && MODE == kMask && m_words > 0) ? (ld_uniform(mrow, 0) & m_valid(0)) : 0u;  // word mw_w + 1
  auto walk = [&](int &lpos, int &mpos) __attribute__((always_inline)) {
    if constexpr (MODE == kDense) {
      lpos = mpos = w_t * kBN;
      ++w_t;
    } else {
      if (w_sub == kSub) {
        w_sub = 0;
        if constexpr (MODE == kList || OSK) {
          ++w_ent;
          w_ok = w_raw >= 0 && w_raw < n_kvblk;
          w_blk = w_ok ? w_raw : 0;
          if (w_ent + 1 < n_ent) w_raw = ld_uniform(crow, w_ent + 1);
        } else {
          while (mw_bits == 0u && mw_w + 1 < m_words) {
            ++mw_w;
            mw_bits = mw_pf;
            mw_pf = mw_w + 1 < m_words ? (ld_uniform(mrow, mw_w + 1) & m_valid(mw_w + 1)) : 0u;
          }
          w_ok = mw_bits != 0u;  // (always, for the counted tiles)
          w_blk = w_ok ? 32 * mw_w + __builtin_ctz(mw_bits) : 0;
          mw_bits &= mw_bits - 1u;
        }
      }
      lpos = w_blk * kListBlock + w_sub * kBN;
      mpos = w_ok ? lpos : kFarKey;
      ++w_sub;
    }
  };
  // pipelined loop, before iteration j: lp[i] is the load position of tile
  // j + i (i < kStages), mp[i] the mask position of tile j - 1 + i (i <= kStages)
  int lp[kStages] = {};
  int mp[kStages + 1] = {};
  if constexpr (kPipe) {
    if (n_iter > 0) {
      walk(lp[0], mp[1]);
      if (loader) issue_rows<C>(smem + kslot(0) + slot_byte0, kt_at(lp[0]), koff, lrow0, k_ssb, len - lp[0]);
    }
  } else {
    kv_cur = n_iter > 0 ? kv_start(0) : -1;
    if (kv_cur >= 0 && loader)
      issue_tile<C>(smem + slot_byte0, smem + kTileBytes + slot_byte0, kt_at(kv_cur), vt_at(kv_cur), koff, voff,
                    lrow0, k_ssb, v_ssb, len - kv_cur);
  }

  // ---- Q rows of this wave, the MFMA B operand (lane l32 holds head-dim
  // values 16*dc + 8*hi .. +7 of its row), loaded after the first K/V tile is
  // issued, so that the two latencies overlap.  The plain kernels load them
  // straight into registers (rows past the end of the sequence read as
  // zero).  The pipelined kernel stages them in this wave's part of the O
  // staging area (free until the epilogue) with whole-row 16 B loads in the
  // K tiles' swizzled layout and reads them into registers after the first
  // barrier: loads in the operand layout touch 32 rows at 32 B each and
  // queue at the texture unit for ~4x as many cache lines.  Rows past the
  // end re-read the last row (finite; never stored).
  bf16x8_t qreg[kDc];
  char *const q_stage = smem + kKVBytes + wave * 32 * L::kRowBytes;
  if constexpr (kPipe) {
    static_assert(kOwnStage, "Q is staged in the O staging area");
    // (an empty block set writes O = 0 through the same area at once: no loads then)
    if (n_iter > 0) {
      stage_q_rows<L::kRowBytes, L::kChunks, L::kRowsPerWin>(q_stage, qg, p.q_ss, w_row0, len, lane);
      // with three slots, K(1) and V(0) behind them (the ring runs two tiles ahead)
      if constexpr (kStages == 3) {
        if (n_iter > 1) {
          walk(lp[1], mp[2]);
          if (loader)
            issue_rows<C>(smem + kslot(1) + slot_byte0, kt_at(lp[1]), koff, lrow0, k_ssb, len - lp[1]);
        }
        if (loader)
          issue_rows<C>(smem + vslot(0) + slot_byte0, vt_at(lp[0]), voff, lrow0, v_ssb, len - lp[0]);
      }
    }
  } else {
    const int r = w_row0 + l32;
#pragma unroll
    for (int dc = 0; dc < kDc; ++dc) {
      uint4_t x = {0u, 0u, 0u, 0u};
      if (r < len) x = ld_global16(qg + (int64_t)r * p.q_ss + dc * 16 + hi * 8);
      qreg[dc] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // Per-lane LDS byte offsets of the MFMA operand reads within a tile.  The
  // swizzles depend only on a row's position within 32 rows (K) and within 4
  // rows (V), so every other read is one of these plus a compile-time row
  // offset.  The empty asm keeps each offset in one register (otherwise the
  // compiler re-splits it into row and chunk parts and re-adds them per read).
  // K: k-step dc reads chunk 2 dc + hi of row l32, stored at chunk
  // (2 dc + hi) ^ swz = (hi ^ swz) ^ 2 dc; the row part of the offset has no
  // bits below the row size, so k-step dc's offset is k-step 0's with dc << 5
  // XORed in.  At head_dim 256 (16 k-steps, one wave per SIMD, where every
  // register counts) the reads form it so, one XOR each; the other head dims
  // keep one register per k-step.
  // V: the pair swizzle takes kPairSwz values, so the offsets of output tiles
  // dt and dt + kPairSwz differ by a constant: kPairSwz registers suffice.
  constexpr bool kKXor = D == 256;
  constexpr int kKRegs = kKXor ? 1 : kDc;
  constexpr int kVRegs = L::kPairSwz < kDt ? L::kPairSwz : kDt;
  int kaddr[kKRegs];
  uint32_t klds[kKRegs], vlds[kVRegs];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_char_t *)smem;
#pragma unroll
  for (int dc = 0; dc < kKRegs; ++dc) {
    kaddr[dc] = L::kq(l32, dc * 2 + hi);
    asm volatile("" : "+v"(kaddr[dc]));
    klds[dc] = smem_lds + (uint32_t)kaddr[dc];
  }
#pragma unroll
  for (int dt = 0; dt < kVRegs; ++dt) {
    int vaddr = L::vv(4 * hi + (j16 >> 2), 2 * dt + (l32 >> 4), (j16 & 3) * 8);
    asm volatile("" : "+v"(vaddr));
    vlds[dt] = smem_lds + (kPipe ? (uint32_t)vslot(0) : 0u) + (uint32_t)vaddr;
  }
  // Offset of k-step dc's K operand from the start of a K tile, given k0 =
  // klds[0] (with kKXor the caller passes a copy made opaque in its own loop
  // body, so that the XORs are not hoisted out into kDc live registers).
  auto k_at = [&](uint32_t k0, int dc) __attribute__((always_inline)) -> uint32_t {
    if constexpr (kKXor) return k0 ^ (uint32_t)(dc << 5);
    else return klds[dc];
  };
  auto k_base = [&]() __attribute__((always_inline)) -> uint32_t {
    uint32_t k0 = klds[0];
    if constexpr (kKXor) asm volatile("" : "+v"(k0));
    return k0;
  };

  // ---- online softmax of one score tile whose first key is kv0 (base 2,
  // scale folded into c): masks the causal diagonal and the sequence tail
  // where the tile needs it, forms P in bf16 in the MFMA operand layout and
  // adds the tile's row sums to l_run.  P is first computed against the
  // running max as it stands; the tile's own max is taken only while some
  // row of the wave has no running max yet (no visible key so far: the
  // wave's first tiles) or when some row sum exceeds kFastSum (a score well
  // above the running max).  Then the max is raised to the tile's, O and l
  // are rescaled and P is computed again.
  bool first = true;  // some row of this wave has seen no visible key yet
  auto mask_tile = [&](floatx16_t (&s)[kKt], const int kv0) __attribute__((always_inline)) {
    const bool need_mask = (kv0 + kBN > len) || (CAUSAL && kv0 + kBN - 1 > w_row0);
    if (need_mask) {
      // key kv0 + hi*4 + o (o a compile-time offset) is masked when o > lim
      const int lim = (CAUSAL ? min(qrow, len - 1) : len - 1) - kv0 - hi * 4;
#pragma unroll
      for (int kt = 0; kt < kKt; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * 32 + (i >> 2) * 8 + (i & 3) > lim) s[kt][i] = -INFINITY;
    }
  };
  // the rest of the online softmax once P has been formed against the
  // running max (row sums rs), or not at all on the wave's first tile
  // (slow): the max raise, O rescale and P again when needed
  auto softmax_slow = [&](floatx16_t (&s)[kKt], bf16x8_t (&pb)[kKt][2], float rs, bool slow) __attribute__((always_inline)) {
    if (slow) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < kKt; ++kt)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(fmaxf(mx, s[kt][i]), s[kt][i + 1]);
      const float mt = half_max(mx) * p.c;
      const bool need = mt > m_run;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? mt : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        m_run = m_new;
        l_run *= alpha;
        if (OSK) d_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) oacc[dt] = oacc[dt] * alpha;
      }
      rs = exp_tile(s, p.c, m_run == -INFINITY ? 0.f : m_run, pb);
      // (a row whose keys were all masked so far keeps m = -inf, and the
      // next tiles must take their max again)
      first = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
    }
    l_run += rs;
    if (OSK) d_run += rs;
  };
  auto softmax = [&](floatx16_t (&s)[kKt], const int kv0, bf16x8_t (&pb)[kKt][2]) __attribute__((always_inline)) {
    mask_tile(s, kv0);
    float rs = 0.f;
    bool slow = first;
    if (!first) {
      rs = exp_tile(s, p.c, m_run == -INFINITY ? 0.f : m_run, pb);
      slow = __builtin_amdgcn_ballot_w64(rs > kFastSum) != 0;
    }
    softmax_slow(s, pb, rs, slow);
  };

  int n_done = n_iter;  // tiles walked (ordered skipping may stop early)
  if constexpr (kPipe) {
   if (n_iter > 0) {
    // ---- software-pipelined loop over a ring of kStages K and V slots.
    // Iteration j (one barrier each, j = 0 .. n_iter) issues the loads of
    // K(j + kStages - 1) and V(j + kStages - 2), and each wave runs one MFMA
    // phase with the scores S(j) = K(j) Q^T interleaved with the PV product
    // of the tile before, O^T += V(j-1)^T P(j-1)^T, and the online softmax of
    // one tile.  K slot t % kStages holds K(t), V slot t % kStages holds
    // V(t); a slot is rewritten one barrier after its last read, and a load
    // has kStages - 1 iterations to land.  Tile positions come from the walk
    // (called once per tile, in order, by every wave).  Waves w, w + 4 (and w + 8)
    // share a SIMD (in the paired block-sparse kernels: the same rows of the
    // two heads); waves 4-7 run the iteration rotated against the others:
    // waves 0-3 (and 8-11) do [MFMA phase][softmax of S(j)], waves 4-7
    // [softmax of S(j-1)][MFMA phase], so that while one wave works through
    // the exp2 and VALU work of the softmax another keeps the matrix core
    // busy.
    const bool lagged = ((wave >> 2) & 1) != 0;
    // tiles this wave needs (dense causal: those not wholly above its rows)
    const int n_own = (CAUSAL && MODE == kDense) ? min(n_iter, wq_last / kBN + 1) : n_iter;
    floatx16_t s[kKt];
    bf16x8_t pb[kKt][2];
    // Before iteration j: K(j) and V(j-1) have landed.  With three slots they
    // were issued one iteration before the loads of iteration j-1, which may
    // stay in flight (2 kLoads per loading wave when that iteration issued
    // both tiles); with two, they are the last loads issued.
    // The barrier is a bare s_barrier (a compiler memory barrier, no fence):
    // the waits above are the ones the ring needs, and a workgroup fence makes
    // the compiler wait for every load in flight (vmcnt(0)) as well.
    auto sync = [&](const int j) __attribute__((always_inline)) {
      if (kStages == 3 && loader && j + 1 < n_iter)
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * C::kLoads));
      else
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      asm volatile("s_barrier" ::: "memory");
    };
    // iteration j's loads: K(j + kStages - 1) (walking on to that tile) and
    // V(j + kStages - 2)
    constexpr int kAhead = kStages - 1;
    auto issue = [&](const int j) __attribute__((always_inline)) {
      if (j + kAhead < n_iter) {
        walk(lp[kAhead], mp[kAhead + 1]);
        if (loader)
          issue_rows<C>(smem + kslot((j + kAhead) % kStages) + slot_byte0, kt_at(lp[kAhead]), koff, lrow0, k_ssb,
                        len - lp[kAhead]);
      }
      if (j + kAhead - 1 < n_iter && loader)
        issue_rows<C>(smem + vslot((j + kAhead - 1) % kStages) + slot_byte0, vt_at(lp[kAhead - 1]), voff, lrow0,
                      v_ssb, len - lp[kAhead - 1]);
    };
    // end of iteration j: tile j + 1 becomes the current one
    auto shift = [&]() __attribute__((always_inline)) {
      static_for<kStages>([&](auto I) { mp[decltype(I)::value] = mp[decltype(I)::value + 1]; });
      static_for<kStages - 1>([&](auto I) { lp[decltype(I)::value] = lp[decltype(I)::value + 1]; });
    };
    int &mp_prv = mp[0];  // mask positions of tiles j - 1 and j
    int &mp_cur = mp[1];
    // One MFMA phase: K from slot kKb, V from slot kVb.  Operand reads run
    // kRing steps ahead of their MFMA; consecutive MFMAs alternate between
    // independent accumulators.
    auto phase = [&](auto kb_tag, auto vb_tag, auto what_tag) __attribute__((always_inline)) {
      constexpr int kKb = decltype(kb_tag)::value;
      constexpr int kVb = decltype(vb_tag)::value;
      constexpr int kW = decltype(what_tag)::value;
      constexpr int kNs = kKt * kDc, kNp = kDt * kKt * 2;
      static_assert(kW != kBoth || kNs == kNp, "score and PV steps must pair up");
      constexpr int kN = kW == kBoth ? kNs + kNp : (kW == kOnlyS ? kNs : kNp);
      constexpr int kRing = 4;
      const uint32_t k0 = k_base();
      auto load = [&](auto T) __attribute__((always_inline)) -> bf16x8_t {
        constexpr int t = decltype(T)::value;
        constexpr int x = step_idx(kW, t);
        if constexpr (step_kind(kW, t) == 0)
          return ld_b128<kKb * kTileBytes + (x % kKt) * 32 * L::kRowBytes>(k_at(k0, x / kKt));
        else
          return tr_pair<kVb * kTileBytes + tr_off<L, kDt>(x) + v_imm<kVRegs>(x % kDt), 8 * L::kRowBytes>(vlds[(x % kDt) % kVRegs]);
      };
      bf16x8_t ring[kRing];
      static_for<kRing>([&](auto T) {
        constexpr int t = decltype(T)::value;
        if constexpr (t < kN) ring[t] = load(T);
      });
      static_for<kN>([&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr int x = step_idx(kW, i);
        lgkm_wait<step_wait(kW, kN, kRing, i)>(ring[i % kRing]);
        if constexpr (step_kind(kW, i) == 0) {
          constexpr int kt = x % kKt, dc = x / kKt;
          if constexpr (dc == 0)
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], qreg[dc], floatx16_t{}, 0, 0, 0);
          else
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], qreg[dc], s[kt], 0, 0, 0);
        } else {
          constexpr int dt = x % kDt, kc = x / kDt;
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], pb[kc >> 1][kc & 1], oacc[dt], 0, 0, 0);
        }
        if constexpr (i + kRing < kN) ring[i % kRing] = load(std::integral_constant<int, i + kRing>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // iteration 0: scores of tile 0 (first Q into registers: this wave's
    // own staging loads have landed)
    sync(0);
    issue(0);
#pragma unroll
    for (int dc = 0; dc < kDc; ++dc)
      qreg[dc] = *reinterpret_cast<const bf16x8_t *>(q_stage + (kKXor ? (kaddr[0] ^ (dc << 5)) : kaddr[dc]));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    phase(BufTag<0>{}, BufTag<0>{}, std::integral_constant<int, kOnlyS>{});
    // Calls body(BufTag<j % kStages>) (the slots of an iteration are
    // compile-time constants, so every LDS operand address is a
    // loop-invariant lane offset plus an immediate).
    auto dispatch = [&](const int j, auto &&body) __attribute__((always_inline)) {
      const int b = j % kStages;
      if (b == 0) body(BufTag<0>{});
      else if (kStages == 2 || b == 1) body(BufTag<1>{});
      else body(BufTag<kStages - 1>{});
    };
    if constexpr (kSolo) {
      // ---- one wave per SIMD: no other wave fills the matrix core while
      // this one runs its softmax, so the softmax is spread over its own
      // MFMAs.  Iteration j forms S(j), then runs O^T += V(j-1)^T P(j-1)^T
      // with the fast-path exp2 of S(j) (against the running max) issued
      // along the PV MFMAs, then finishes the softmax of S(j) (the rare max
      // raise and O rescale come after the PV MFMAs that precede them).
      // P(j) goes to P buffer j % 3 (the slot index of its tile).
      constexpr int kNpv = kDt * kKt * 2;          // PV MFMAs per tile
      constexpr int kE = kKt * 16 / kNpv;          // exp2 issued per PV MFMA
      static_assert(kE * kNpv == kKt * 16, "the scores of a tile spread evenly over its PV MFMAs");
      bf16x8_t pp[kStages][kKt][2];
      softmax(s, mp_cur, pp[0]);
      shift();
      auto pv_exp = [&](auto vb_tag, auto ps_tag, auto pd_tag) __attribute__((always_inline)) -> float {
        constexpr int kVb = decltype(vb_tag)::value;  // V slot of the PV tile
        constexpr int kPs = decltype(ps_tag)::value;  // its P buffer
        constexpr int kPd = decltype(pd_tag)::value;  // P buffer of S (-1: no exp2)
        constexpr int kN = kNpv;
        constexpr int kRing = 4;
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float rs = 0.f;
        auto load = [&](auto T) __attribute__((always_inline)) -> bf16x8_t {
          constexpr int t = decltype(T)::value;
          return tr_pair<kVb * kTileBytes + tr_off<L, kDt>(t) + v_imm<kVRegs>(t % kDt), 8 * L::kRowBytes>(vlds[(t % kDt) % kVRegs]);
        };
        bf16x8_t ring[kRing];
        static_for<kRing>([&](auto T) { ring[decltype(T)::value] = load(T); });
        static_for<kN>([&](auto I) {
          constexpr int i = decltype(I)::value;
          constexpr int dt = i % kDt, kc = i / kDt;
          lgkm_wait<2 * (kN - 1 - i < kRing - 1 ? kN - 1 - i : kRing - 1)>(ring[i % kRing]);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], pp[kPs][kc >> 1][kc & 1], oacc[dt], 0, 0, 0);
          if constexpr (i + kRing < kN) ring[i % kRing] = load(std::integral_constant<int, i + kRing>{});
          if constexpr (kPd >= 0) {
            static_for<kE>([&](auto E) {
              constexpr int e = i * kE + decltype(E)::value;  // score e % 16 of tile e / 16
              float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e / 16][e % 16], p.c, -m_use));
              // (the volatile asm pins the exp2 here: on a wave's first tiles its
              // result is dropped for the slow path's, and the compiler would
              // otherwise move all of them into a branch after the MFMAs)
              asm volatile("" : "+v"(pv));
              rs += pv;
              pp[kPd][e / 16][(e % 16) >> 3][e & 7] = (__bf16)pv;
            });
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        return rs;
      };
      int j = 1;
      auto body_solo = [&](auto kb_tag) __attribute__((always_inline)) {
        constexpr int kKb = decltype(kb_tag)::value;  // = j % kStages: K slot and P buffer of tile j
        constexpr int kVb = (kKb + kStages - 1) % kStages;
        sync(j);
        issue(j);
        phase(kb_tag, BufTag<kVb>{}, std::integral_constant<int, kOnlyS>{});
        mask_tile(s, mp_cur);
        const float rs = pv_exp(BufTag<kVb>{}, BufTag<kVb>{}, BufTag<kKb>{});
        softmax_slow(s, pp[kKb], rs, first || __builtin_amdgcn_ballot_w64(rs > kFastSum) != 0);
        shift();
        ++j;
      };
      // iterations 1 .. n_own - 1, kStages per trip (j % kStages = 1, .., 0)
      while (j + kStages - 1 < n_own) {
        static_for<kStages>([&](auto I) { body_solo(BufTag<(decltype(I)::value + 1) % kStages>{}); });
      }
      static_for<kStages - 1>([&](auto I) {
        if (j < n_own) body_solo(BufTag<decltype(I)::value + 1>{});
      });
      // iteration n_own: PV of the wave's last tile
      sync(n_own);
      issue(n_own);
      auto last_solo = [&](auto vb_tag) __attribute__((always_inline)) { pv_exp(vb_tag, vb_tag, BufTag<-1>{}); };
      dispatch(n_own - 1, last_solo);
      shift();
      for (int jj = n_own + 1; jj <= n_iter; ++jj) {
        sync(jj);
        issue(jj);
        shift();
      }
    } else {
      // Ordered skipping (paired kernel): end_h[x] is the last tile whose
      // scores head x counts (x = 0: waves 0-3; x = 1: the lagged waves 4-7),
      // n_iter - 1 until the head stops.  A head's waves post their stop flags
      // after the softmax of an entry's last tile (head 1 one iteration later
      // than head 0, being lagged) and every wave reads them after the next
      // barrier, so both heads' decisions are the same in every wave.  A
      // stopped head still runs the PV of its last tile (in the iteration
      // after it), then only joins the barriers and the loads; the workgroup
      // leaves the loop at the start of an iteration (its loads all landed)
      // once both heads are past their last PV.
      int end_h[2] = {n_iter - 1, n_iter - 1};
      const int hx = lagged ? 1 : 0;
      bool quit = false;
      // after the softmax of tile t: at an entry's end, this wave's flag (all
      // its rows pass: the entries still to come, if each adds at most what
      // this one added, would add at most tau of the row's mass)
      auto osk_mark = [&](const int t) __attribute__((always_inline)) {
        if constexpr (OSK) {
          if (t % kSub != kSub - 1) return;
          const float share = half_sum(d_run);
          const float mass = half_sum(l_run);
          const float left = (float)(n_ent - (t / kSub + 1));  // entries not yet visited
          const bool fail = __builtin_amdgcn_ballot_w64(left * share > p.osk_tau * mass) != 0;
          if (lane == 0) osk_flag[wave] = fail ? 0u : 1u;
          // (the loop's barrier is a bare s_barrier: the flag must be written first)
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          d_run = 0.f;
        }
      };
      // after the barrier of iteration j: the heads' decisions (head 0 on the
      // entry that ended with tile j - 1, head 1 on the one that ended with
      // tile j - 2)
      auto osk_check = [&](const int j) __attribute__((always_inline)) {
        if constexpr (OSK) {
          if (j < n_iter) {
            if (end_h[0] == n_iter - 1 && j % kSub == 0 && j / kSub >= p.osk_min_visit &&
                (osk_flag[0] & osk_flag[1] & osk_flag[2] & osk_flag[3]))
              end_h[0] = j - 1;
            if (end_h[1] == n_iter - 1 && j % kSub == 1 && (j - 1) / kSub >= p.osk_min_visit &&
                (osk_flag[4] & osk_flag[5] & osk_flag[6] & osk_flag[7]))
              end_h[1] = j - 2;
          }
          quit = j >= max(end_h[0], end_h[1]) + 2;
        }
      };
      if (!lagged) {
        softmax(s, mp_cur, pb);
        osk_mark(0);
      }
      shift();
      int j = 1;
      auto body = [&](auto kb_tag) __attribute__((always_inline)) {
        constexpr int kKb = decltype(kb_tag)::value;  // = j % kStages
        constexpr int kVb = (kKb + kStages - 1) % kStages;
        if constexpr (OSK) {
          if (quit) return;
          sync(j);
          osk_check(j);
          if (quit) return;
          issue(j);
          const int e = end_h[hx];
          if (lagged && j - 1 <= e) {
            softmax(s, mp_prv, pb);
            osk_mark(j - 1);
          }
          // (with the PV of a stopped head's last tile comes the scores of
          // the next one, which it never uses: one phase, one copy of its code)
          if (j - 1 <= e) phase(kb_tag, BufTag<kVb>{}, std::integral_constant<int, kBoth>{});
          if (!lagged && j <= e) {
            softmax(s, mp_cur, pb);
            osk_mark(j);
          }
        } else {
          sync(j);
          issue(j);
          if (lagged) softmax(s, mp_prv, pb);
          phase(kb_tag, BufTag<kVb>{}, std::integral_constant<int, kBoth>{});
          if (!lagged) softmax(s, mp_cur, pb);
        }
        shift();
        ++j;
      };
      // iterations 1 .. n_own - 1, kStages per trip (j % kStages = 1, .., 0)
      while (j + kStages - 1 < n_own && !quit) {
        static_for<kStages>([&](auto I) { body(BufTag<(decltype(I)::value + 1) % kStages>{}); });
      }
      static_for<kStages - 1>([&](auto I) {
        if (j < n_own) body(BufTag<decltype(I)::value + 1>{});
      });
      if (!quit) {
        // iteration n_own: PV of the wave's last tile
        sync(n_own);
        issue(n_own);
        const int e = OSK ? end_h[hx] : n_own - 1;
        if (lagged && n_own - 1 <= e) softmax(s, mp_prv, pb);
        auto last = [&](auto vb_tag) __attribute__((always_inline)) {
          phase(BufTag<0>{}, vb_tag, std::integral_constant<int, kOnlyPV>{});
        };
        if (n_own - 1 <= e) dispatch(n_own - 1, last);
        shift();
        // the other waves' remaining iterations: barriers and loads only
        for (int jj = n_own + 1; jj <= n_iter; ++jj) {
          sync(jj);
          issue(jj);
          shift();
        }
      }
      if constexpr (OSK) n_done = end_h[hx] + 1;
    }
   }
  } else {
    // Returns true (ordered skipping only) when the walk stops before tile `it`.
    auto step = [&](const int it, auto buf_tag) -> bool {
      constexpr int kBuf = decltype(buf_tag)::value;  // LDS buffer of tile `it` (= it % 2)
      // tile `it` has landed (every wave waited for its own loads); every wave is
      // done reading the other buffer
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      // ordered skipping: at the start of a list entry, stop when every wave found
      // all its rows' share of the previous entry at most tau of their mass
      if (OSK && it > 0 && it % kSub == 0 && it / kSub >= p.osk_min_visit &&
          (osk_flag[0] & osk_flag[1] & osk_flag[2] & osk_flag[3]))
        return true;
      int kv_nxt = -1;
      if (it + 1 < n_iter) {
        kv_nxt = kv_start(it + 1);
        if (kv_nxt >= 0) {
          char *buf = smem + (1 - kBuf) * kBufBytes;
          issue_tile<C>(buf + slot_byte0, buf + kTileBytes + slot_byte0, kt_at(kv_nxt), vt_at(kv_nxt), koff, voff,
                        lrow0, k_ssb, v_ssb, len - kv_nxt);
        }
      }
      const int kv0 = kv_cur;
      kv_cur = kv_nxt;
      if (kv0 < 0) return false;
      if (CAUSAL && kv0 > wq_last) return false;  // whole tile above this wave's rows

      // ---- S^T = K Q^T : kKt tiles of 32 keys x 32 query rows
      floatx16_t s[kKt];
      {
        // LDS operand reads run kRing MFMAs ahead of their use, each waited for
        // exactly (reads complete in order), and consecutive MFMAs alternate
        // between the kKt independent accumulators, so neither the LDS
        // latency nor the MFMA dependency latency is exposed
        constexpr int kRing = 4;
        constexpr int kSteps = kKt * kDc;  // step i: kt = i % kKt, dc = i / kKt
        const uint32_t k0 = k_base();
        auto load = [&](auto T) __attribute__((always_inline)) -> bf16x8_t {
          constexpr int t = decltype(T)::value;
          return ld_b128<kBuf * kBufBytes + (t % kKt) * 32 * L::kRowBytes>(k_at(k0, t / kKt));
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

      bf16x8_t pb[kKt][2];
      softmax(s, kv0, pb);

      // ---- O^T += V^T P^T.  MFMA k index (8 per lane half) maps to keys
      // 16c + 8(e/4) + 4*hi + (e%4) of a 32-key tile, matching where the score
      // layout left P; V^T operands are read with the LDS transpose.
      {
        // same operand ring as for S; consecutive MFMAs alternate between the
        // kDt output accumulators
        constexpr int kRing = 4;
        constexpr int kSteps = kDt * kKt * 2;  // step i: dt = i % kDt, (kt, c) = i / kDt
        constexpr int kVOff = kBuf * kBufBytes + kTileBytes;  // V tile of this buffer
        bf16x8_t ring[kRing];
        static_for<kRing>([&](auto I) {
          constexpr int i = decltype(I)::value;
          ring[i] = tr_pair<kVOff + tr_off<L, kDt>(i) + v_imm<kVRegs>(i % kDt), 8 * L::kRowBytes>(vlds[(i % kDt) % kVRegs]);
        });
        static_for<kSteps>([&](auto I) {
          constexpr int i = decltype(I)::value;
          constexpr int dt = i % kDt, kc = i / kDt, kt = kc >> 1, c = kc & 1;
          // the reads of step i are done once at most the reads issued after
          // them are outstanding (LDS reads complete in order)
          lgkm_wait<2 * (kSteps - 1 - i < kRing - 1 ? kSteps - 1 - i : kRing - 1)>(ring[i % kRing]);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kRing], pb[kt][c], oacc[dt], 0, 0, 0);
          if constexpr (i + kRing < kSteps)
            ring[i % kRing] = tr_pair<kVOff + tr_off<L, kDt>(i + kRing) + v_imm<kVRegs>((i + kRing) % kDt), 8 * L::kRowBytes>(
                vlds[((i + kRing) % kDt) % kVRegs]);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      return false;
    };
    // ordered skipping: after the last tile of a list entry, each wave records
    // whether all its rows passed the test -- the entries still to come, if
    // each adds at most what this one added, would add at most tau of the
    // row's mass -- and starts the next entry's share
    auto osk_mark = [&](const int it) {
      if (!OSK || it % kSub != kSub - 1) return;
      const float share = half_sum(d_run);
      const float mass = half_sum(l_run);
      const float left = (float)(n_iter / kSub - (it / kSub + 1));  // entries not yet visited
      const bool fail = __builtin_amdgcn_ballot_w64(left * share > p.osk_tau * mass) != 0;
      if (lane == 0) osk_flag[wave] = fail ? 0u : 1u;
      d_run = 0.f;
    };
    // two tiles per trip so that each step's LDS buffer is a compile-time constant
    // (every LDS operand address is then a loop-invariant lane offset plus an
    // immediate)
    for (int it = 0; it < n_iter; it += 2) {
      if (step(it, BufTag<0>{})) {
        n_done = it;
        break;
      }
      osk_mark(it);
      if (it + 1 < n_iter) {
        if (step(it + 1, BufTag<1>{})) {
          n_done = it + 1;
          break;
        }
        osk_mark(it + 1);
      }
    }
  }
  if (OSK && p.visited && lane == 0 && wave % kWph == 0) p.visited[(int64_t)h * p.n_tiles + tile] = n_done / kSub;

  // ---- epilogue: O = acc / l (bf16, round to nearest even), LSE in natural log.
  // O goes out through LDS: each wave writes its 32 x D tile there (16 B
  // chunks XOR-swizzled by row) and reads it back so that 16 consecutive
  // lanes store one whole row with 16-byte stores (the accumulator layout
  // would otherwise store 8 bytes per lane into 32 different rows at a time).
  const float l_tot = half_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (!kOwnStage) __syncthreads();  // every wave is done with the K/V buffers
  {
    constexpr int kRowB = D * 2;           // bytes per O row
    constexpr int kCh = D / 8;             // 16 B chunks per row
    constexpr int kRowsPerStore = 1024 / kRowB;
    char *so = smem + (kOwnStage ? kKVBytes : 0) + wave * 32 * kRowB;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const floatx2_t f01 = {oacc[dt][g4 * 4 + 0] * inv, oacc[dt][g4 * 4 + 1] * inv};
        const floatx2_t f23 = {oacc[dt][g4 * 4 + 2] * inv, oacc[dt][g4 * 4 + 3] * inv};
        uint2_t w;
        w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f01, bf16x2_t));
        w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(f23, bf16x2_t));
        const int ch = (dt * 4 + g4) ^ (l32 % kCh);
        *reinterpret_cast<uint2_t *>(so + l32 * kRowB + ch * 16 + hi * 8) = w;
      }
    constexpr int kStores = 32 / kRowsPerStore;
    const int r0 = lane / kCh;  // row (within the wave's 32) of this lane's first store
    const int ch = lane % kCh;
    uint4_t x[kStores];
#pragma unroll
    for (int k = 0; k < kStores; ++k) {
      const int r = k * kRowsPerStore + r0;
      x[k] = *reinterpret_cast<const uint4_t *>(so + r * kRowB + ((ch ^ (r % kCh)) * 16));
    }
    uint16_t *orow = og + (int64_t)(w_row0 + r0) * p.o_ss + ch * 8;
    const int64_t step_rows = (int64_t)kRowsPerStore * p.o_ss;
    if (w_row0 + 32 <= len) {
#pragma unroll
      for (int k = 0; k < kStores; ++k) *reinterpret_cast<uint4_t *>(orow + k * step_rows) = x[k];
    } else {
#pragma unroll
      for (int k = 0; k < kStores; ++k)
        if (w_row0 + k * kRowsPerStore + r0 < len)
          *reinterpret_cast<uint4_t *>(orow + k * step_rows) = x[k];
    }
  }
  if (qrow < len) {
    if (p.lse && hi == 0) {
      const float v = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
      int64_t idx;
      if (p.cu) {
        const int64_t total = p.cu[p.batch];
        idx = (int64_t)h * total + tok0 + qrow;
      } else {
        idx = ((int64_t)b * p.hq + h) * p.seqlen + qrow;
      }
      p.lse[idx] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
bool stride_ok(int64_t s) { return ((s * 2) % 16) == 0; }
// K and V row strides: the kernels address a tile's rows with 32-bit byte
// offsets from the tile's first row
constexpr int64_t kMaxKvRowStride = int64_t(1) << 24;  // elements

int validate(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
             const int32_t *cu_seqlens, int causal, float scale, const attn_block_list_t *bl,
             const attn_tensor_t *out) {
  if (!q || !k || !v || !out) return ATTN_ERR_INVALID_ARG;
  const attn_tensor_t *all[4] = {q, k, v, out};
  for (const attn_tensor_t *t : all) {
    if (t->batch < 0 || t->seqlen < 0 || t->heads < 1 || t->head_dim < 1)
      return ATTN_ERR_INVALID_ARG;
  }
  if (k->batch != q->batch || v->batch != q->batch || out->batch != q->batch)
    return ATTN_ERR_INVALID_ARG;
  if (k->seqlen != q->seqlen || v->seqlen != q->seqlen || out->seqlen != q->seqlen)
    return ATTN_ERR_INVALID_ARG;
  if (k->head_dim != q->head_dim || v->head_dim != q->head_dim || out->head_dim != q->head_dim)
    return ATTN_ERR_INVALID_ARG;
  if (k->heads != v->heads || out->heads != q->heads || q->heads % k->heads != 0)
    return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (bl) {
    if (!bl->row_ptr || !bl->col_idx) return ATTN_ERR_INVALID_ARG;
    if (bl->block_q != kListBlock || bl->block_k != kListBlock) return ATTN_ERR_UNSUPPORTED;
    if (cu_seqlens || q->batch > 1) return ATTN_ERR_UNSUPPORTED;
    if (bl->num_q_blocks != (q->seqlen + kListBlock - 1) / kListBlock) return ATTN_ERR_INVALID_ARG;
  }
  const bool empty = q->batch == 0 || q->seqlen == 0;
  if (!empty) {
    for (const attn_tensor_t *t : all)
      if (!t->data) return ATTN_ERR_INVALID_ARG;
  }
  const int d = q->head_dim;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
  if (!(scale > 0.f)) return ATTN_ERR_UNSUPPORTED;
  for (const attn_tensor_t *t : all) {
    if (!aligned16(t->data)) return ATTN_ERR_UNSUPPORTED;
    if (!stride_ok(t->stride_seq) || !stride_ok(t->stride_head)) return ATTN_ERR_UNSUPPORTED;
    if (!cu_seqlens && !stride_ok(t->stride_batch)) return ATTN_ERR_UNSUPPORTED;
  }
  for (const attn_tensor_t *t : {k, v})
    if (t->stride_seq < 0 || t->stride_seq >= kMaxKvRowStride) return ATTN_ERR_UNSUPPORTED;
  if (!empty) {
    const int64_t tiles = (q->seqlen + 127) / 128;
    if (tiles * (int64_t)q->batch * q->heads > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
  }
  return ATTN_OK;
}

template <class C, bool CAUSAL, int MODE>
int launch(Params p, hipStream_t stream) {
  // query heads per workgroup: two for the paired block-list / block-mask kernels
  const int hpw = (MODE == kList || MODE == kMask || MODE == kOsk) && C::NW == 8 ? 2 : 1;
  const int rows = C::kBM / hpw;
  p.n_tiles = (p.seqlen + rows - 1) / rows;
  p.n_units = p.batch * (p.hq / hpw);
  p.unit_group = p.group / hpw;
  p.xcd_remap = (p.n_units % (8 * p.unit_group)) == 0 ? 1 : 0;
  const int64_t n_blocks = (int64_t)p.n_tiles * p.n_units;
  constexpr int64_t kCUs = 256;  // compute units of an MI355X
  p.group_major = n_blocks >= 8 * kCUs ? 1 : 0;  // at least 8 workgroups per CU
  if ((MODE == kList || MODE == kMask) && p.group_major) p.group_major = 2;
  void *args[] = {&p};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&attn_fwd_kernel<C, CAUSAL, MODE>),
                                 dim3((unsigned)n_blocks), dim3(C::kThreads), args, 0, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

constexpr float kOskPairedMaxTau = 1e-2f;  // ordered skipping: the paired kernel up to this tau

template <int D>
int launch_d(const Params &p, bool causal, int mode, hipStream_t s) {
  using Dense = Config<D, D == 64 ? 12 : (D == 128 ? 8 : 4)>;
  using Listed = Config<D, 4>;
  // Block list and block mask: two query heads of one GQA group per workgroup
  // when the group splits in pairs (head_dim 256: one head, four waves, in the
  // solo form of the pipelined loop); else the plain four-wave kernel.
  using Paired = Config<D, D == 256 ? 4 : 8>;
  const bool paired = D == 256 || p.group % 2 == 0;
  if (mode == kList) {
    if (paired) return causal ? launch<Paired, true, kList>(p, s) : launch<Paired, false, kList>(p, s);
    return causal ? launch<Listed, true, kList>(p, s) : launch<Listed, false, kList>(p, s);
  }
  if (mode == kMask) {
    if (paired) return causal ? launch<Paired, true, kMask>(p, s) : launch<Paired, false, kMask>(p, s);
    return causal ? launch<Listed, true, kMask>(p, s) : launch<Listed, false, kMask>(p, s);
  }
  if (mode == kOsk) {
    // Two heads per workgroup when most of each list is walked.  With a larger
    // tau the walks are short, a pair's per-workgroup cost weighs more and the
    // pair waits for its slower head (128K planted-relevance workload: the
    // paired kernel 5-7% faster at tau <= 1e-3, even at 3e-3 and 1e-2, 2-3%
    // slower at 3e-2 and 1e-1).  Head_dim 256 and odd groups: one head per
    // workgroup, plain loop.
    if (D != 256 && p.group % 2 == 0 && p.osk_tau <= kOskPairedMaxTau)
      return causal ? launch<Paired, true, kOsk>(p, s) : launch<Paired, false, kOsk>(p, s);
    return causal ? launch<Listed, true, kOsk>(p, s) : launch<Listed, false, kOsk>(p, s);
  }
  return causal ? launch<Dense, true, kDense>(p, s) : launch<Dense, false, kDense>(p, s);
}

// Checks of attn_fwd_mask beyond those of attn_fwd.
int validate_mask(const attn_tensor_t *q, const attn_block_mask_t *m) {
  if (!m) return ATTN_ERR_INVALID_ARG;
  if (m->block_q != kListBlock || m->block_k != kListBlock) return ATTN_ERR_UNSUPPORTED;
  if (m->stride_seq < 0 || m->stride_head < 0) return ATTN_ERR_INVALID_ARG;
  const int64_t n_blk = (q->seqlen + kListBlock - 1) / kListBlock;
  if (m->num_q_blocks < n_blk || (int64_t)m->words_per_row * 32 < n_blk || m->words_per_row < 1)
    return ATTN_ERR_INVALID_ARG;
  if (q->batch > 0 && q->seqlen > 0 && !m->bits) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

Params make_params(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                   const int32_t *cu_seqlens, float scale, attn_tensor_t *out, float *lse) {
  Params p;
  p.q = static_cast<const uint16_t *>(q->data);
  p.k = static_cast<const uint16_t *>(k->data);
  p.v = static_cast<const uint16_t *>(v->data);
  p.o = static_cast<uint16_t *>(out->data);
  p.lse = lse;
  p.q_sb = q->stride_batch; p.q_ss = q->stride_seq; p.q_sh = q->stride_head;
  p.k_sb = k->stride_batch; p.k_ss = k->stride_seq; p.k_sh = k->stride_head;
  p.v_sb = v->stride_batch; p.v_ss = v->stride_seq; p.v_sh = v->stride_head;
  p.o_sb = out->stride_batch; p.o_ss = out->stride_seq; p.o_sh = out->stride_head;
  p.cu = cu_seqlens;
  p.row_ptr = nullptr;
  p.col_idx = nullptr;
  p.mask = nullptr;
  p.mask_ss = p.mask_sh = 0;
  p.mask_words = 0;
  p.osk_tau = 0.f;
  p.osk_min_visit = 1;
  p.visited = nullptr;
  p.batch = q->batch;
  p.seqlen = q->seqlen;
  p.hq = q->heads;
  p.group = q->heads / k->heads;
  p.n_tiles = p.n_units = p.unit_group = p.xcd_remap = p.group_major = 0;  // set per configuration at launch
  p.c = scale * 1.44269504088896340736f;
  return p;
}

int launch_any(const Params &p, int d, bool causal, int mode, hipStream_t s) {
  switch (d) {
    case 64: return launch_d<64>(p, causal, mode, s);
    case 128: return launch_d<128>(p, causal, mode, s);
    default: return launch_d<256>(p, causal, mode, s);
  }
}

}  // namespace

extern "C" int attn_fwd_validate(const attn_tensor_t *q, const attn_tensor_t *k,
                                 const attn_tensor_t *v, const int32_t *cu_seqlens, int causal,
                                 float scale, const attn_block_list_t *block_list,
                                 const attn_tensor_t *out) {
  return validate(q, k, v, cu_seqlens, causal, scale, block_list, out);
}

extern "C" int attn_fwd(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                        const int32_t *cu_seqlens, int causal, float scale,
                        const attn_block_list_t *block_list, attn_tensor_t *out, float *lse,
                        void *stream) {
  const int st = validate(q, k, v, cu_seqlens, causal, scale, block_list, out);
  if (st != ATTN_OK) return st;
  if (q->batch == 0 || q->seqlen == 0) return ATTN_OK;
  Params p = make_params(q, k, v, cu_seqlens, scale, out, lse);
  if (block_list) {
    p.row_ptr = block_list->row_ptr;
    p.col_idx = block_list->col_idx;
  }
  return launch_any(p, q->head_dim, causal, block_list ? kList : kDense,
                    static_cast<hipStream_t>(stream));
}

extern "C" int attn_fwd_mask_validate(const attn_tensor_t *q, const attn_tensor_t *k,
                                      const attn_tensor_t *v, const int32_t *cu_seqlens,
                                      int causal, float scale, const attn_block_mask_t *mask,
                                      const attn_tensor_t *out) {
  const int st = validate(q, k, v, cu_seqlens, causal, scale, nullptr, out);
  if (st != ATTN_OK) return st;
  return validate_mask(q, mask);
}

extern "C" int attn_fwd_mask(const attn_tensor_t *q, const attn_tensor_t *k,
                             const attn_tensor_t *v, const int32_t *cu_seqlens, int causal,
                             float scale, const attn_block_mask_t *mask, attn_tensor_t *out,
                             float *lse, void *stream) {
  const int st = attn_fwd_mask_validate(q, k, v, cu_seqlens, causal, scale, mask, out);
  if (st != ATTN_OK) return st;
  if (q->batch == 0 || q->seqlen == 0) return ATTN_OK;
  Params p = make_params(q, k, v, cu_seqlens, scale, out, lse);
  p.mask = mask->bits;
  p.mask_ss = mask->stride_seq;
  p.mask_sh = mask->stride_head;
  p.mask_words = mask->words_per_row;
  return launch_any(p, q->head_dim, causal, kMask, static_cast<hipStream_t>(stream));
}

extern "C" int attn_fwd_osk_validate(const attn_tensor_t *q, const attn_tensor_t *k,
                                     const attn_tensor_t *v, int causal, float scale,
                                     const attn_block_list_t *block_list, float tau,
                                     int min_visit, const attn_tensor_t *out) {
  if (!block_list) return ATTN_ERR_INVALID_ARG;
  const int st = validate(q, k, v, nullptr, causal, scale, block_list, out);
  if (st != ATTN_OK) return st;
  if (!isfinite(tau) || tau < 0.f || min_visit < 1) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

extern "C" int attn_fwd_osk(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                            int causal, float scale, const attn_block_list_t *block_list,
                            float tau, int min_visit, attn_tensor_t *out, float *lse,
                            int32_t *visited, void *stream) {
  const int st = attn_fwd_osk_validate(q, k, v, causal, scale, block_list, tau, min_visit, out);
  if (st != ATTN_OK) return st;
  if (q->batch == 0 || q->seqlen == 0) return ATTN_OK;
  Params p = make_params(q, k, v, nullptr, scale, out, lse);
  p.row_ptr = block_list->row_ptr;
  p.col_idx = block_list->col_idx;
  p.osk_tau = tau;
  p.osk_min_visit = min_visit;
  p.visited = visited;
  return launch_any(p, q->head_dim, causal, kOsk, static_cast<hipStream_t>(stream));
}

extern "C" const char *attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported argument combination";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_TOO_LARGE: return "problem exceeds the library's static scratch buffer";
    default: return "unknown status";
  }
}

extern "C" int attn_version(void) { return 301; }

#ifndef ATTN_SOURCE_SHA
#define ATTN_SOURCE_SHA "unknown"
#endif
extern "C" const char *attn_source_sha(void) { return ATTN_SOURCE_SHA; }
