// Forward pass of exact tiled attention for gfx950.
//
// What is computed: O = softmax(scale * Q K^T [causal mask]) V and the
// natural-log logsumexp of each row of scaled scores (FlashAttention-2
// abstract on the "High-Bandwidth Memory" keyword page; IPLEX post on
// FlashAttention-2 GPU work partitioning, section "Tiling preserves the
// attention calculation": tiles on chip, running statistics and rescaled
// partial outputs, no full score matrix stored).
//
// Work partitioning (same post, section "Three changes improve GPU
// utilisation"): one workgroup per (query block of 128 rows, head, batch),
// so long sequences with few heads still fill the chip; inside a workgroup
// each of the 4 wavefronts owns 32 query rows and all of them share the K/V
// tiles staged in LDS, so no partial results are exchanged between waves.
// Two (d = 128) or three to four (d = 64) workgroups share a CU, so one wave's
// softmax arithmetic overlaps another's matrix instructions; a d = 128
// launch too small for that (at most one workgroup per CU) gives each
// workgroup two groups of 4 waves that split the key tiles between them and
// combine their partial results at the end. Self-attention launches at
// d = 128 over at least 2048 keys with more than a round of work take
// fwd48_kernel instead: 192-row workgroups of four 48-row waves, two per CU
// (see there).
//
// K/V tiles move from memory straight into LDS with buffer loads
// that write LDS directly (no register staging), double-buffered: the next
// tile streams in while the current one is used. Rows past the end of the
// sequence come back as zeros from the buffer range check.
//
// Per wave and K/V tile of 64 keys:
//   S^T = K Q^T     (MFMA; lane l owns query row l % 32, so a row's scores
//                    sit in two lanes: l and l ^ 32)
//   online softmax in the log2 domain: c2 = |scale| * log2(e) is folded into
//   one FMA per score before exp2; the running sum stays per lane until the
//   epilogue; the division by the row sum is deferred to the epilogue; and
//   the running max (with the rescale of the partial output) is only moved
//   when a probability relative to it would exceed 2^8, which keeps every
//   exponent <= 8 while skipping almost all rescales. That test needs no row
//   maximum: P is taken from the current running max and each lane's sum of
//   it compared with 2^8; only a tile that fails it (rare after the first)
//   forms the row maxima (one cross-half exchange) and takes P again.
//   O^T += V^T P^T  (MFMA; P^T is taken straight from the S^T accumulator
//                    registers, V^T is read with LDS transpose loads)
// Causal masking: tiles entirely above the diagonal are never visited, and a
// wave skips tiles that are fully masked for its 32 rows; only tiles that
// straddle the diagonal (or the ragged end of the sequence) apply a mask.
// A negative softmax scale is handled by negating Q when it is loaded.

#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

// Per head dimension: query rows per workgroup (32 per wave), keys per K/V
// tile, LDS stages of the K/V ring and waves per SIMD. Both use 128 rows
// (4 waves) per workgroup and a double-buffered ring. d = 64 runs three
// workgroups per CU on 64-key tiles (its softmax work per matrix instruction
// is twice that of d = 128, so a third wave hides more of it; 64-key rather
// than 32-key tiles halve its per-tile fixed work). d = 128 also runs three,
// on 32-key tiles: 64-key ones take 64 KiB of LDS per workgroup, which
// leaves room for only two, and a third wave per SIMD gains more than the
// larger tiles' lower fixed work (measured 0.5-4% faster on causal 2k-16k
// launches, the same non-causal). With a bias, d = 128 keeps 64-key tiles
// and two workgroups per CU (its bias staging does not fit three). (256-row
// workgroups and deeper rings were measured slower: one workgroup per CU
// leaves each workgroup's start and end exposed.)
template <int D_, int BR_, int BC_, int STAGES_, int WAVES_PER_SIMD_>
struct KernelCfg {
  static constexpr int D = D_, BR = BR_, BC = BC_, STAGES = STAGES_, WAVES_PER_SIMD = WAVES_PER_SIMD_;
  static constexpr int KSPLIT = 1;  // groups of waves that share a query block (below)
  static constexpr int GROUP_ROUNDS = 2;  // block order: XCD rounds of blocks per head group
};
template <int D> struct FwdCfg;
template <> struct FwdCfg<64> : KernelCfg<64, 128, 64, 2, 3> {};
template <> struct FwdCfg<128> : KernelCfg<128, 128, 32, 2, 3> {};
template <int D> struct FwdBiasCfg : FwdCfg<D> {};
template <> struct FwdBiasCfg<128> : KernelCfg<128, 128, 64, 2, 2> {};
// d = 64 without a bias fits four workgroups per CU (128 registers, 32 KiB
// of LDS each). Measured faster for key lengths up to 4096 (short and
// mid-length sequences: more waves to hide the softmax, whole rounds of
// workgroups) and slower at 16384 (more workgroups share each L2), so the
// launch picks it by key length.
struct FwdCfg64Short : KernelCfg<64, 128, 64, 2, 4> {};
constexpr int kFwd64ShortMaxKeys = 4096;
// A launch of at most one workgroup per CU (e.g. one 2048-row chunk of 16
// heads) would leave a single wave per SIMD, so no second wave would hide
// one wave's softmax behind another's matrix instructions. Such launches use
// workgroups of 8 waves in two groups of 4 over the same 128 query rows: the
// first group takes the even K/V tiles of the key range and the second the
// odd ones, each with its own LDS ring, so every SIMD runs two waves. At the
// end the second group hands its running max, row sums and partial output to
// the first through LDS, which combines the two exactly (each part rescaled
// to the larger max) and writes the result. (Measured 9-21% faster on such
// launches than one group that overlaps the next tile's scores with the
// current tile's softmax inside each wave.)
struct FwdCfgSplit128 : KernelCfg<128, 128, 64, 2, 2> {
  static constexpr int KSPLIT = 2;
};
constexpr int kNumCus = kNumXcd * kCusPerXcd;
// Query rows per workgroup of fwd48_kernel (4 waves x 48 rows), and the
// shortest sequence it takes (launch_fwd).
constexpr int kFwd48Rows = 192;
constexpr int kFwd48MinKeys = 2048;
// Decode-shaped calls (a few query rows against a long key history) are
// bound by streaming K and V from memory, and their parallelism comes from
// splitting the keys, not from query blocks: one wave per workgroup holds
// all (up to 32) query rows of a (batch, head) and streams one key range.
// d = 64 keeps two tiles in flight per wave (3 stages; its tiles are half
// the size), d = 128 one (measured best).
template <int D> struct DecCfg;
template <> struct DecCfg<64> : KernelCfg<64, 32, kDecodeBC, 3, 2> {
  static constexpr int GROUP_ROUNDS = 1;
};
template <> struct DecCfg<128> : KernelCfg<128, 32, kDecodeBC, 2, 2> {
  static constexpr int GROUP_ROUNDS = 1;
};
constexpr float kRescaleSlack = 8.f;  // log2 units a row max may exceed the running max
constexpr float kPSumMax = 256.f;     // 2^kRescaleSlack
// The running max of a row that has seen no key: finite, so that P taken
// from it is +inf for any visible score and exactly 0 for a masked one.
constexpr float kNoMax = -1e30f;

// Nq query rows attend to Nk key rows. With the causal mask key j is visible
// to query i iff j <= i + delta (delta = global position of query row 0 minus
// that of key row 0; 0 for plain self-attention). F32OUT: O is written as
// float32 (a chunk result that a merge combines later), otherwise bfloat16.
// The keys may be split into nsplit ranges of split_len keys (a multiple of
// the tile width), one workgroup each; split s writes its result at
// O + s * o_split and LSE + s * l_split (elements).
// BIAS: bfloat16 additive bias on the scaled scores, element (b, h, i, j) at
// Bias[b * bias_sb + h * bias_sh + i * bias_srow + j] (bias_srow a multiple
// of 8, the row base 16-byte aligned); keys past Nk are always masked so the
// padding of a bias row is never used.
template <typename Cfg, bool CAUSAL, bool F32OUT, bool BIAS = false>
__global__ __launch_bounds__(Cfg::BR * 2 * Cfg::KSPLIT)
__attribute__((amdgpu_waves_per_eu(Cfg::WAVES_PER_SIMD, Cfg::WAVES_PER_SIMD))) void fwd_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    void* __restrict__ O, float* __restrict__ LSE, int Nq, int Nk, int delta, int H, int nqb,
    int nsplit, int split_len, long o_split, long l_split, int total_blocks, float c2, uint32_t q_sign,
    const bf16* __restrict__ Bias = nullptr, long bias_sb = 0, long bias_sh = 0, int bias_srow = 0) {
  constexpr int D = Cfg::D;                        // head dimension
  constexpr int kFwdBR = Cfg::BR;                  // query rows per workgroup
  constexpr int kFwdBC = Cfg::BC;                  // keys per K/V tile
  constexpr int STAGES = Cfg::STAGES;              // K/V tiles in the LDS ring
  constexpr int NW = kFwdBR / 32;                  // waves per group (one per 32 query rows)
  constexpr int KSPLIT = Cfg::KSPLIT;              // groups of waves, each with every KSPLIT-th tile
  static_assert(KSPLIT == 1 || !BIAS, "split groups: no bias");
  constexpr int KB = kFwdBC / 32;                  // 32-key score blocks per tile
  using T = Tile<kFwdBC, D>;                       // one K or V tile in LDS
  constexpr int TILE = T::BYTES;
  static_assert(T::LOADS % NW == 0 || NW % T::LOADS == 0, "tile loads split evenly over the waves");
  constexpr int DMA_PER_WAVE = (T::LOADS + NW - 1) / NW;  // 1 KiB wave loads per tile per wave and tensor
  constexpr int KS = D / 16;                       // MFMA k-steps over d
  constexpr int DB = D / 32;                       // 32-wide output column blocks
  // Per group and stage: K tile, V tile. With several groups the same memory
  // later holds the partial results of groups 1.. for the combine (NX floats
  // per lane).
  constexpr int NX = D / 32 * 16 + 2;
  constexpr int RING = KSPLIT * STAGES * 2 * TILE;
  constexpr int XCHG = (KSPLIT - 1) * NW * NX * 64 * 4;
  __shared__ __attribute__((aligned(1024))) char ring[RING > XCHG ? RING : XCHG];
  // Bias of the next tile for each wave's 32 rows (see bias_fetch below).
  __shared__ __attribute__((aligned(BIAS ? 1024 : 16))) char bias_lds[BIAS ? NW * 32 * kFwdBC * 2 : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int half = KSPLIT > 1 ? wave_id / NW : 0;  // this wave's group: tiles j0 + half, + KSPLIT, ...
  const int wave = wave_id - half * NW;            // query rows 32 * wave .. of the block
  const int g = lane >> 5, l32 = lane & 31, G = lane >> 4;
  char* const ring_h = ring + half * (STAGES * 2 * TILE);

  const HeadRank hr = block_order<CAUSAL>(blockIdx.x, total_blocks / (nqb * nsplit), nqb * nsplit,
                                          kCusPerXcd * Cfg::WAVES_PER_SIMD / KSPLIT, Cfg::GROUP_ROUNDS);
  const int head = hr.head;                        // b * H + h
  const int qblk = nqb - 1 - hr.rank / nsplit;     // longest causal rows first
  const int split = hr.rank - (hr.rank / nsplit) * nsplit;
  const int b = head / H, h = head - b * H;
  const long hq = ((long)b * Nq * H + h) * D;      // element offset of query / output token 0
  const long hk = ((long)b * Nk * H + h) * D;      // element offset of key / value token 0
  const uint32_t tokb = (uint32_t)H * D * 2;       // bytes between tokens
  const auto rq = make_rsrc(Q + hq, (uint32_t)(Nq - 1) * tokb + D * 2);
  const uint32_t nrec_k = Nk > 0 ? (uint32_t)(Nk - 1) * tokb + D * 2 : 0u;
  const u32x4 rk = make_raw_rsrc(K + hk, nrec_k);
  const u32x4 rv = make_raw_rsrc(V + hk, nrec_k);

  const int qw0 = qblk * kFwdBR + wave * 32;       // first query row of this wave
  const int myq = qw0 + l32;
  // The last key this lane's row sees (masked tiles: one compare per score).
  const int key_lim = CAUSAL ? min(myq + delta, Nk - 1) : Nk - 1;

  // Bias rows of this (batch, head), each bias_srow elements of readable
  // memory (the 8-byte loads of a row's last keys reach into its padding);
  // rows at or past Nq read as zeros.
  const auto rb = make_rsrc(BIAS ? Bias + b * bias_sb + h * bias_sh : Q,
                            BIAS ? (uint32_t)((long)Nq * bias_srow * 2) : 0u);

  // Q as the B operand of S^T = K Q^T: row myq, d = 16*ks + 8*g .. +7.
  bf16x8 qf[KS];
  {
    const uint32_t qoff = row_off(myq, Nq, tokb, 16 * g);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, qoff + 32 * ks) ^ q_sign);
  }

  // LDS-DMA: wave load u = wave + NW t of a tile; lane i fills the chunk
  // (row, column) the layout assigns to it. A tile row is a key. The lane's
  // byte offset inside a tile is fixed; the tile's position goes into the
  // (scalar) resource, whose end still turns rows past Nk into zeros.
  uint32_t dma_off[DMA_PER_WAVE];
#pragma unroll
  for (int t = 0; t < DMA_PER_WAVE; ++t) {
    const int u = min(wave + NW * t, T::LOADS - 1);
    dma_off[t] = (uint32_t)T::dma_row(u, lane) * tokb + 16u * T::dma_chunk(u, lane);
  }
  const uint32_t ring_lds = lds_base(ring_h);
  auto issue = [&](int tile, char* dst, int t0 = 0, int t1 = 1 << 20) __attribute__((always_inline)) {
    const uint32_t toff = (uint32_t)(tile * kFwdBC) * tokb;
    const u32x4 rkt = rsrc_advance(rk, toff), rvt = rsrc_advance(rv, toff);
    const uint32_t l0 = ring_lds + (uint32_t)(dst - ring_h);
#pragma unroll
    for (int t = 0; t < DMA_PER_WAVE; ++t) {
      if (t < t0 || t >= t1) continue;
      const int u = wave + NW * t;
      if (T::LOADS < NW && u >= T::LOADS) break;  // fewer loads than waves: the rest issue none
      dma16_at(rkt, l0 + T::dma_dst(u), dma_off[t]);
      dma16_at(rvt, l0 + T::dma_dst(u) + TILE, dma_off[t]);
    }
  };

  // Keys up to the last one visible to the block's last row, within this
  // workgroup's key range [k_lo, k_lo + split_len): tiles j0 .. j1 - 1.
  const int kv_len = CAUSAL ? max(0, min(Nk, (qblk + 1) * kFwdBR + delta)) : Nk;
  const int k_lo = split * split_len;
  const int k_end = min(kv_len, k_lo + split_len);
  const int j0 = k_lo / kFwdBC;
  const int j1 = k_end > k_lo ? (k_end + kFwdBC - 1) / kFwdBC : j0;
  const int ntiles = j1 - j0;
  // This group's tiles: j0 + KSPLIT * t + half for t < nth; all groups run
  // nit iterations (one barrier each), a group without a tile idles in it.
  const int nit = (ntiles + KSPLIT - 1) / KSPLIT;
  const int nth = max(0, (ntiles - half + KSPLIT - 1) / KSPLIT);

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = kNoMax;     // running max of c2 * score (log2 domain), possibly stale by <= 8
  float l_run = 0.f;        // this lane's share of the running sum

  // One K/V tile. MASK selects the variant for tiles that straddle the
  // causal diagonal or the end of the sequence; all other tiles run the
  // variant without any per-element masking.
  // Bias of a tile for the wave's 32 rows (32 x kFwdBC bf16): fetched with
  // 16-byte loads that cover whole rows (each load instruction reads
  // 64 / CH full rows) into registers, written to the wave's own LDS slice
  // (row r, 16-byte chunk c at slot c ^ (r % CH)), and read back in the
  // accumulator layout: per 32-key block, 4 groups of 4 consecutive keys
  // (the keys of the lane's accumulator rows), 8 bytes each. A lane of the
  // accumulator layout holds one query row, so reading the bias in that
  // layout straight from memory touches 32 rows per load instruction.
  constexpr int CH = kFwdBC / 8;        // 16-byte chunks per bias row of a tile
  constexpr int RB = kFwdBC * 2;        // bytes per bias row of a tile
  constexpr int BL = 32 * CH / 64;      // 16-byte loads per lane and tile
  char* const bw_lds = bias_lds + wave * 32 * RB;
  uint32_t bgo[BIAS ? BL : 1];          // per-lane global byte offsets at key 0
  if constexpr (BIAS) {
#pragma unroll
    for (int t = 0; t < BL; ++t) {
      const int row = t * (64 / CH) + lane / CH, chunk = lane % CH;
      bgo[t] = ((uint32_t)min(qw0 + row, Nq) * (uint32_t)bias_srow + 8u * chunk) * 2u;
    }
  }
  u32x4 bst[BIAS ? BL : 1];
  auto bias_fetch = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < BL; ++t)
      bst[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(bgo[t] + (uint32_t)(j * RB)), 0, 0));
  };
  auto bias_store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < BL; ++t) {
      const int row = t * (64 / CH) + lane / CH, chunk = lane % CH;
      lds_write16(bw_lds, row * RB + ((chunk ^ (row % CH)) << 4), bst[t]);
    }
  };
  // The scores of a tile: S^T = K Q^T for the wave's rows, then (with a
  // bias) c2 * s + bias * log2(e), then the mask.
  auto scores = [&](f32x16 (&s)[KB], const char* kt, int key0, auto mask_tag, auto&& mid)
                    __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    u32x2 bw[BIAS ? KB : 1][4];
    if constexpr (BIAS) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int c = kb * 4 + rg;
          bw[kb][rg] = *reinterpret_cast<const FA_LDS u32x2*>(
              (const FA_LDS char*)bw_lds + l32 * RB + ((c ^ (l32 % CH)) << 4) + 8 * g);
        }
    }
    // The KB accumulation chains are interleaved (independent MFMAs back to back).
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = mfma32(T::row8(kt, kb * 32 + l32, 2 * ks + g), qf[ks], s[kb]);
    mid();  // the rest of the next tile's loads (after this tile's S product)
    // With a bias the scores become log2-domain values here, c2 * s + bias * log2(e).
    if constexpr (BIAS) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = __builtin_fmaf(s[kb][r], c2, bf16_elem(bw[kb][r >> 2], r & 3) * kLog2e);
    }
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key > key_lim) s[kb][r] = -INFINITY;
        }
    }
  };
  // P = exp2(c2 s - m) (with a bias exp2(s - m)) in bf16 for the PV product;
  // returns this lane's fp32 sum of the tile's P (the row sum stays in fp32:
  // the logsumexp is checked against the exact value, so it must not inherit
  // the bf16 rounding of P).
  auto probs = [&](const f32x16 (&s)[KB], float m, bf16x8 (&pf)[2 * KB], auto mask_tag)
                   __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    float t = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2 * KB; ++ks) {
      f32x8 p;
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) {
        const float sv = s[ks >> 1][8 * (ks & 1) + s8];
        float e;
        if constexpr (BIAS) {
          e = fast_exp2(sv - m);  // -inf (masked or a -inf bias) gives exactly 0
        } else {
          e = fast_exp2(__builtin_fmaf(sv, c2, -m));
          if constexpr (MASK) e = (sv == -INFINITY) ? 0.f : e;  // exact zero even when c2 = 0
        }
        p[s8] = e;
      }
      t += sum8(p);
      pf[ks] = to_bf16x8(p);
    }
    return t;
  };
  // One K/V tile. MASK selects the variant for tiles that straddle the
  // causal diagonal or the end of the sequence; all other tiles run the
  // variant without any per-element masking.
  // The running max m_run only has to move when a probability relative to
  // it would exceed 2^8 (kRescaleSlack). The tile's P is first taken from
  // the current m_run; since P >= 0, a lane whose sum of the tile's P stays
  // <= 2^8 has every value <= 2^8, so if no lane of the wave exceeds that,
  // P stands and the tile needs no row maximum at all. Otherwise (and on
  // the first tile) the scores are formed again (the first pass consumed
  // them; the K tile and the tile's bias are still in LDS), the row maxima
  // taken, m_run moved to them, O and l rescaled, and P recomputed. A row
  // that has seen no key has m_run = kNoMax, for which every visible score
  // overflows to +inf and takes the second path. (The d = 64 bias form
  // keeps the per-tile maximum: the registers of both paths do not fit its
  // three waves per SIMD.)
  constexpr bool FAST = !BIAS || D == 128;
  auto compute = [&](int j, const char* kt, auto mask_tag, auto&& mid, bool first) __attribute__((always_inline)) {
    const int key0 = j * kFwdBC;
    const char* vt = kt + TILE;
    f32x16 s[KB];
    scores(s, kt, key0, mask_tag, mid);
    bf16x8 pf[2 * KB];
    float t = 0.f;
    bool slow = true;  // wave-uniform
    if (FAST && !first) {
      t = probs(s, m_run, pf, mask_tag);
      slow = __builtin_amdgcn_ballot_w64(!(t <= kPSumMax)) != 0;
    }
    if (slow) {
      asm volatile("" ::: "memory");  // a branch; the scores below are loaded again
      if (FAST && !first) scores(s, kt, key0, mask_tag, []() {});
      float mx = max16(s[0], -INFINITY);
#pragma unroll
      for (int kb = 1; kb < KB; ++kb) mx = max16(s[kb], mx);
      mx = xhalf_max(mx);
      const float tile_m = (mx == -INFINITY) ? -INFINITY : (BIAS ? mx : mx * c2);
      // The second path moves m_run to the tile's maximum (the d = 64 bias
      // form, which has no first path, keeps the slack rule).
      const bool grow = FAST ? tile_m > m_run : tile_m > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {  // wave-uniform
        asm volatile("" ::: "memory");          // keep it a branch (no speculation)
        const float m_new = grow ? tile_m : m_run;
        const float alpha = fast_exp2(m_run - m_new);  // 0 from kNoMax, 1 when unchanged
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        m_run = m_new;
      }
      t = probs(s, m_run, pf, mask_tag);
    }
    l_run += t;
#pragma unroll
    for (int ks = 0; ks < 2 * KB; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 a = T::col8(vt, 16 * ks + 4 * g, 16 * ks + 8 + 4 * g, 32 * db + 16 * (G & 1), lane);
        oacc[db] = mfma32(a, pf[ks], oacc[db]);
      }
  };
  // The t-th tile of a group (tile j0 + KSPLIT * t + half) lives in stage
  // t % STAGES of the group's ring. Iteration t first refills the stage that
  // its tile t - 1 used (every wave finished it before the last barrier)
  // with its tile t + STAGES - 1, computes tile t, then waits for its own
  // loads of tile t + 1 (the loads of later tiles may stay in flight) and
  // meets the other waves at the barrier, after which tile t + 1 is complete
  // in LDS.
  auto stage = [&](int t) __attribute__((always_inline)) { return ring_h + (t % STAGES) * (2 * TILE); };
  static_assert(STAGES >= 2 && STAGES <= 4, "K/V ring depth");
  auto wait_next = [&](int t) __attribute__((always_inline)) {
    if constexpr (STAGES >= 4) {
      if (t + 3 < nth) {  // tiles t + 2 and t + 3 may stay in flight
        wait_vmem_leave<4 * DMA_PER_WAVE>();
        return;
      }
    }
    if constexpr (STAGES >= 3) {
      if (t + 2 < nth) {  // tile t + 2 may stay in flight
        wait_vmem_leave<2 * DMA_PER_WAVE>();
        return;
      }
    }
    wait_vmem();
  };
  // Tiles before jm need no mask for any wave of this workgroup; they run in
  // a loop of their own so that the masked variant never joins the hot loop.
  // (causal: the tiles whose last key is visible to the block's first row)
  const int jm_all = CAUSAL ? min(max(0, qblk * kFwdBR + delta + 1) / kFwdBC, Nk / kFwdBC) : Nk / kFwdBC;
  const int jm = min(max(jm_all, j0), j1);
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t)
    if (t < nth) issue(j0 + KSPLIT * t + half, stage(t));
  if (BIAS && j0 < j1) bias_fetch(j0);
  wait_next(-1);
  if (BIAS && j0 < j1) bias_store();
  __syncthreads();
  int t = 0;
  // In the unmasked causal loop half of a wave's loads of the next tile are
  // issued before this tile's S product and half after it, so the LDS
  // writes of the workgroup's loads do not arrive in one burst (long causal
  // loops have the latency to spare; short non-causal ones do not).
  // With a bias, iteration j also fetches the bias of tile j + 1 into
  // registers and writes it to the wave's LDS slice after this tile's
  // compute has read tile j's (a wave's LDS operations run in order).
  constexpr int SPLIT = CAUSAL ? DMA_PER_WAVE / 2 : DMA_PER_WAVE;
  // Unmasked iterations: every group's tile lies before jm.
  const int tu = (jm - j0) / KSPLIT;
  constexpr int AHEAD = KSPLIT * (STAGES - 1);  // tile distance of a refill
  for (; t < tu; ++t) {
    const int j = j0 + KSPLIT * t + half;
    const bool more = t + STAGES - 1 < nth;
    if (more) issue(j + AHEAD, stage(t + STAGES - 1), 0, SPLIT);
    if (BIAS && j + 1 < j1) bias_fetch(j + 1);
    compute(
        j, stage(t), std::false_type{},
        [&]() __attribute__((always_inline)) {
          if (SPLIT < DMA_PER_WAVE && more) issue(j + AHEAD, stage(t + STAGES - 1), SPLIT, DMA_PER_WAVE);
        },
        t == 0);
    wait_next(t);
    if (BIAS && j + 1 < j1) bias_store();
    __syncthreads();
  }
  for (; t < nit; ++t) {
    const int j = j0 + KSPLIT * t + half;
    if (t + STAGES - 1 < nth) issue(j + AHEAD, stage(t + STAGES - 1));
    if (BIAS && j + 1 < j1) bias_fetch(j + 1);
    // A tile whose first key lies past this wave's last row is fully masked
    // for it and contributes nothing (and a group may have no tile left).
    if (t < nth && (!CAUSAL || j * kFwdBC <= qw0 + 31 + delta)) compute(j, stage(t), std::true_type{}, []() {}, t == 0);
    wait_next(t);
    if (BIAS && j + 1 < j1) bias_store();
    __syncthreads();
  }

  if constexpr (KSPLIT > 1) {
    // Combine the groups. The loops end at a barrier, so the rings are free:
    // each group h >= 1 stores, per lane, its partial output, running max and
    // row-sum share (element i of wave w's lane at float
    // ((h - 1) * NW + w) * NX * 64 + i * 64 + lane: conflict-free); a lane of
    // group 0 holds the same row and keys of the same layout. Every part is
    // rescaled to the largest max; a part that saw no key (max kNoMax) counts 0.
    static_assert(NX == DB * 16 + 2, "exchange record: output, max, row sum");
    FA_LDS float* const xs = (FA_LDS float*)ring + wave * NX * 64 + lane;
    constexpr int XG = NW * NX * 64;  // floats per group
    if (half > 0) {
      FA_LDS float* const mine = xs + (half - 1) * XG;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(db * 16 + r) * 64] = oacc[db][r];
      mine[DB * 16 * 64] = m_run;
      mine[(DB * 16 + 1) * 64] = l_run;
    }
    __syncthreads();
    if (half > 0) return;
    float m = m_run;
#pragma unroll
    for (int p = 0; p < KSPLIT - 1; ++p) m = fmaxf(m, xs[p * XG + DB * 16 * 64]);
    const float a0 = fast_exp2(m_run - m);  // 0 for a part that saw no key (kNoMax)
    l_run *= a0;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= a0;
    float ap[KSPLIT - 1];
#pragma unroll
    for (int p = 0; p < KSPLIT - 1; ++p) {
      const float mp = xs[p * XG + DB * 16 * 64];
      ap[p] = fast_exp2(mp - m);
      l_run += xs[p * XG + (DB * 16 + 1) * 64] * ap[p];
    }
    // One 32-column block at a time (keeps the loads in flight few).
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int p = 0; p < KSPLIT - 1; ++p)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] += xs[p * XG + (db * 16 + r) * 64] * ap[p];
      __builtin_amdgcn_sched_barrier(0);
    }
    m_run = m;
  }

  // A row that saw no key (possible only with a causal offset that puts every
  // key after it) has l = 0: its output is 0 and its logsumexp -inf.
  const float l_tot = xhalf_sum(l_run);
  const bool seen = l_tot > 0.f;
  const float inv = seen ? 1.f / l_tot : 0.f;
  if (myq < Nq) {
    if (g == 0) LSE[split * l_split + (long)head * Nq + myq] = seen ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    const long row = split * o_split + hq + (long)myq * H * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq4 = 0; rq4 < 4; ++rq4) {
        f32x4 x = {oacc[db][4 * rq4] * inv, oacc[db][4 * rq4 + 1] * inv, oacc[db][4 * rq4 + 2] * inv,
                   oacc[db][4 * rq4 + 3] * inv};
        const int col = 32 * db + 8 * rq4 + 4 * g;
        if constexpr (F32OUT)
          *reinterpret_cast<f32x4*>(static_cast<float*>(O) + row + col) = x;
        else
          *reinterpret_cast<bf16x4*>(static_cast<bf16*>(O) + row + col) = to_bf16x4(x);
      }
  }
}

// Self-attention at d = 128 (bf16 output, no bias): 48 query rows per wave
// on 16x16x32 MFMAs, 4 waves (192 rows) per workgroup sharing each K/V tile,
// two workgroups per CU. Every K and V^T operand read from LDS feeds three
// MFMAs (one per 16-row query block of the wave), and every K/V tile brought
// into LDS serves 192 rows: a third fewer LDS and LDS-DMA bytes per flop than
// 32-row waves in 128-row workgroups, at the cost of the third wave per SIMD
// (48 rows need ~240 registers).
//
// Per wave and 32-key tile:
//   S^T = K Q^T  as 2 x 3 blocks of 16 keys x 16 query rows (lane l owns
//                query column l % 16 of each block and keys 4G .. 4G+3,
//                G = l / 16; a row's 32 scores sit in four lanes)
//   online softmax in the log2 domain with the sum test of fwd_kernel, per
//                query block (three running maxima and sums per lane)
//   O^T += V^T P^T  as 8 x 3 blocks of 16 columns x 16 rows: P^T is taken
//                straight from the S^T accumulators (keys 4G .. 4G+3 of the
//                two 16-key blocks as the k slots 8G .. 8G+7), V^T with LDS
//                transpose reads of the same keys.
// Causal blocks are aligned to the end of the sequence, so the one partial
// block is the lightest (rows before 0 are absent: their Q reads as zeros,
// every key is masked for them, nothing of theirs is stored); non-causal
// blocks start at row 0 and the last one is partial.
template <bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd48_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V, bf16* __restrict__ O,
    float* __restrict__ LSE, int N, int H, int nqb, int total_blocks, float c2, uint32_t q_sign) {
  constexpr int D = 128, NW = 4, WR = kFwd48Rows / NW, QB = WR / 16;
  constexpr int BC = 32, KB = BC / 16, DS = D / 32, DB = D / 16, STAGES = 2;
  using T = Tile<BC, D, true>;  // the swizzle under which the K and V^T reads below are conflict-free
  constexpr int TILE = T::BYTES;
  constexpr int DMA_PER_WAVE = T::LOADS / NW;
  static_assert(T::LOADS % NW == 0, "tile loads split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char ring[STAGES * 2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int G = lane >> 4, c16 = lane & 15;
  const HeadRank hr = block_order<CAUSAL>(blockIdx.x, total_blocks / nqb, nqb, kCusPerXcd * 2, 2);
  const int head = hr.head, qblk = nqb - 1 - hr.rank;  // longest causal rows first
  const int b = head / H, h = head - b * H;
  const long hoff = ((long)b * N * H + h) * D;
  const uint32_t tokb = (uint32_t)H * D * 2;
  const uint32_t nrec = (uint32_t)(N - 1) * tokb + D * 2;
  const auto rq = make_rsrc(Q + hoff, nrec);
  const u32x4 rk = make_raw_rsrc(K + hoff, nrec), rv = make_raw_rsrc(V + hoff, nrec);

  const int row0 = CAUSAL ? N - (nqb - qblk) * kFwd48Rows : qblk * kFwd48Rows;
  const int qw0 = row0 + wave * WR;  // first query row of this wave (may be < 0)
  // Q as the B operand: query block qb, row qw0 + 16 qb + c16, d = 32 ds + 8G .. +7.
  bf16x8 qf[QB][DS];
  int key_lim[QB];  // the last key each of the lane's rows sees
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + 16 * qb + c16;
    key_lim[qb] = CAUSAL ? min(row, N - 1) : N - 1;
    const uint32_t off = (uint32_t)((row < 0 || row >= N) ? N : row) * tokb + 16u * G;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[qb][ds] = __builtin_bit_cast(bf16x8, buf_load16(rq, off + 64 * ds) ^ q_sign);
  }

  // LDS-DMA of a tile as in fwd_kernel: fixed per-lane offsets, the tile's
  // position in the scalar resource.
  uint32_t dma_off[DMA_PER_WAVE];
#pragma unroll
  for (int t = 0; t < DMA_PER_WAVE; ++t) {
    const int u = wave + NW * t;
    dma_off[t] = (uint32_t)T::dma_row(u, lane) * tokb + 16u * T::dma_chunk(u, lane);
  }
  const uint32_t ring_lds = lds_base(ring);
  auto issue = [&](int tile) __attribute__((always_inline)) {
    const uint32_t toff = (uint32_t)(tile * BC) * tokb;
    const u32x4 rkt = rsrc_advance(rk, toff), rvt = rsrc_advance(rv, toff);
    const uint32_t l0 = ring_lds + (uint32_t)((tile % STAGES) * 2 * TILE);
#pragma unroll
    for (int t = 0; t < DMA_PER_WAVE; ++t) {
      const int u = wave + NW * t;
      dma16_at(rkt, l0 + T::dma_dst(u), dma_off[t]);
      dma16_at(rvt, l0 + T::dma_dst(u) + TILE, dma_off[t]);
    }
  };

  // Tiles 0 .. ntiles - 1; those before tu need no mask for any row of the block.
  const int kv_len = CAUSAL ? max(0, min(N, row0 + kFwd48Rows)) : N;
  const int ntiles = (kv_len + BC - 1) / BC;
  const int tu = min(CAUSAL ? min(max(0, row0 + 1) / BC, N / BC) : N / BC, ntiles);

  f32x4 oacc[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = f32x4{};
  float m_run[QB], l_run[QB];  // per query block: running max (log2 domain, stale by <= 8), lane's sum share
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) m_run[qb] = kNoMax, l_run[qb] = 0.f;

  auto compute = [&](int j, const char* kt, auto mask_tag, bool first) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* vt = kt + TILE;
    const int key0 = j * BC;
    f32x4 s[KB][QB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x4{};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = T::row8(kt, 16 * kb + c16, 4 * ds + G);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma16(a, qf[qb][ds], s[kb][qb]);
      }
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key0 + 16 * kb + 4 * G + i > key_lim[qb]) s[kb][qb][i] = -INFINITY;
    }
    // P^T in bf16 (k slots 8G .. 8G+7 = keys 4G .. 4G+3 of both 16-key
    // blocks) and the lane's fp32 sums of P per query block.
    bf16x8 pf[QB];
    float t[QB];
    auto probs = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x8 p;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sv = s[e >> 2][qb][e & 3];
          float x = fast_exp2(__builtin_fmaf(sv, c2, -m_run[qb]));
          if constexpr (MASK) x = (sv == -INFINITY) ? 0.f : x;  // exact zero even when c2 = 0
          p[e] = x;
        }
        t[qb] = sum8(p);
        pf[qb] = to_bf16x8(p);
      }
    };
    // The sum test of fwd_kernel, for all three query blocks at once; the
    // scores stay in registers for the second path.
    bool slow = true;  // wave-uniform
    if (!first) {
      probs();
      slow = __builtin_amdgcn_ballot_w64(!(t[0] <= kPSumMax && t[1] <= kPSumMax && t[2] <= kPSumMax)) != 0;
    }
    if (slow) {
      asm volatile("" ::: "memory");  // a branch
      bool grow[QB], any = false;
      float tile_m[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mx = vmax3(mx, vmax(s[kb][qb][0], s[kb][qb][1]), vmax(s[kb][qb][2], s[kb][qb][3]));
        mx = xquad_max(mx);
        tile_m[qb] = (mx == -INFINITY) ? -INFINITY : mx * c2;
        grow[qb] = tile_m[qb] > m_run[qb];
        any |= grow[qb];
      }
      if (__builtin_amdgcn_ballot_w64(any)) {  // wave-uniform
        asm volatile("" ::: "memory");        // keep it a branch (no speculation)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float m_new = grow[qb] ? tile_m[qb] : m_run[qb];
          const float alpha = fast_exp2(m_run[qb] - m_new);  // 0 from kNoMax, 1 when unchanged
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
          m_run[qb] = m_new;
        }
      }
      probs();
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += t[qb];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = T::col8(vt, 4 * G, 16 + 4 * G, 16 * db, lane);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = mfma16(a, pf[qb], oacc[db][qb]);
    }
  };

  // Double-buffered ring: iteration t loads tile t + 1 into the stage tile
  // t - 1 used (every wave finished it before the last barrier), computes
  // tile t, waits for its own loads and meets the other waves at the barrier.
  if (ntiles > 0) issue(0);
  wait_vmem();
  __syncthreads();
  int t = 0;
  for (; t < tu; ++t) {
    if (t + 1 < ntiles) issue(t + 1);
    compute(t, ring + (t % STAGES) * 2 * TILE, std::false_type{}, t == 0);
    wait_vmem();
    __syncthreads();
  }
  for (; t < ntiles; ++t) {
    if (t + 1 < ntiles) issue(t + 1);
    // A causal tile whose first key lies past this wave's last row is fully masked for it.
    if (!CAUSAL || t * BC <= qw0 + WR - 1) compute(t, ring + (t % STAGES) * 2 * TILE, std::true_type{}, t == 0);
    wait_vmem();
    __syncthreads();
  }

  // A row that saw no key (only causal rows before 0) has l = 0 and is not stored.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = xquad_sum(l_run[qb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int row = qw0 + 16 * qb + c16;
    if (row >= 0 && row < N) {
      if (G == 0) LSE[(long)head * N + row] = l_tot > 0.f ? (m_run[qb] + log2f(l_tot)) * kLn2 : -INFINITY;
      bf16* const orow = O + hoff + (long)row * H * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<bf16x4*>(orow + 16 * db + 4 * G) = to_bf16x4(oacc[db][qb] * inv);
    }
  }
}

}  // namespace

template <int D, bool CAUSAL>
hipError_t launch_fwd(const FwdArgs& a) {
  constexpr int BR = FwdCfg<D>::BR;
  static_assert(FwdBiasCfg<D>::BR == BR, "one block size per head dimension");
  const int nqb = (a.Nq + BR - 1) / BR;
  const int total = a.B * a.H * nqb;
  const float c2 = fabsf(a.scale) * kLog2e;
  const uint32_t q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  const auto* q = static_cast<const bf16*>(a.q);
  const auto* k = static_cast<const bf16*>(a.k);
  const auto* v = static_cast<const bf16*>(a.v);
  if (a.bias) {
    hipLaunchKernelGGL((fwd_kernel<FwdBiasCfg<D>, CAUSAL, false, true>), dim3(total), dim3(BR * 2), 0, a.stream, q, k,
                       v, a.o, a.lse, a.Nq, a.Nk, a.delta, a.H, nqb, 1, a.Nk, 0L, 0L, total, c2, q_sign,
                       static_cast<const bf16*>(a.bias), a.bias_sb, a.bias_sh, a.bias_srow);
    return hipGetLastError();
  }
  auto plain = [&](auto cfg) {
    using Cfg = decltype(cfg);
    static_assert(Cfg::BR == BR, "one block size per head dimension");
    const dim3 block(BR * 2 * Cfg::KSPLIT);
    if (a.f32_out)
      hipLaunchKernelGGL((fwd_kernel<Cfg, CAUSAL, true>), dim3(total), block, 0, a.stream, q, k, v, a.o, a.lse,
                         a.Nq, a.Nk, a.delta, a.H, nqb, 1, a.Nk, 0L, 0L, total, c2, q_sign);
    else
      hipLaunchKernelGGL((fwd_kernel<Cfg, CAUSAL, false>), dim3(total), block, 0, a.stream, q, k, v, a.o, a.lse,
                         a.Nq, a.Nk, a.delta, a.H, nqb, 1, a.Nk, 0L, 0L, total, c2, q_sign);
  };
  if constexpr (D == 64) {
    if (a.Nk <= kFwd64ShortMaxKeys)
      plain(FwdCfg64Short{});
    else
      plain(FwdCfg<D>{});
  } else {
    // Self-attention over at least 2048 keys with more than one round of
    // 192-row workgroups (two per CU) takes fwd48_kernel. Measured against
    // the 128-row kernel: causal 1-8% faster (B=4 H=16 N=4096 262 -> 239 us,
    // N = 16384 974 -> 864 us), non-causal 1-2.5% faster; with one round or
    // less it was 4-15% slower (the heaviest blocks set the time), and below
    // 2048 keys equal to 12% slower (short rows: the per-block start and the
    // rounding of the block count to whole rounds weigh more).
    const int nqb48 = (a.Nq + kFwd48Rows - 1) / kFwd48Rows;
    const int total48 = a.B * a.H * nqb48;
    if (total <= kNumCus) {
      plain(FwdCfgSplit128{});
    } else if (!a.f32_out && a.delta == 0 && a.Nq == a.Nk && a.Nq >= kFwd48MinKeys && total48 > 2 * kNumCus) {
      hipLaunchKernelGGL(fwd48_kernel<CAUSAL>, dim3(total48), dim3(256), 0, a.stream, q, k, v,
                         static_cast<bf16*>(a.o), a.lse, a.Nq, a.H, nqb48, total48, c2, q_sign);
    } else {
      plain(FwdCfg<D>{});
    }
  }
  return hipGetLastError();
}

// Decode: the keys are split into ranges (decode_split); each range's result
// goes to the float32 workspace and the merge combines them into o and lse.
// With a single range the kernel writes o (bf16) and lse directly.
template <int D, bool CAUSAL>
hipError_t launch_decode(const DecodeArgs& a) {
  using Cfg = DecCfg<D>;
  const DecodeSplit sp = decode_split(a.B, a.Nq, a.Nk, a.H, D);
  const int nqb = (a.Nq + Cfg::BR - 1) / Cfg::BR;
  const int total = a.B * a.H * nqb * sp.nsplit;
  const float c2 = fabsf(a.scale) * kLog2e;
  const uint32_t q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  const auto* q = static_cast<const bf16*>(a.q);
  const auto* k = static_cast<const bf16*>(a.k);
  const auto* v = static_cast<const bf16*>(a.v);
  if (sp.nsplit == 1) {
    hipLaunchKernelGGL((fwd_kernel<Cfg, CAUSAL, false>), dim3(total), dim3(Cfg::BR * 2), 0, a.stream, q, k, v,
                       a.o, a.lse, a.Nq, a.Nk, a.delta, a.H, nqb, 1, sp.split_len, 0L, 0L, total, c2, q_sign);
    return hipGetLastError();
  }
  const long rows = (long)a.B * a.Nq * a.H;
  float* o_parts = a.workspace;
  float* l_parts = a.workspace + decode_part_elems((long)sp.nsplit * rows * D);
  hipLaunchKernelGGL((fwd_kernel<Cfg, CAUSAL, true>), dim3(total), dim3(Cfg::BR * 2), 0, a.stream, q, k, v,
                     o_parts, l_parts, a.Nq, a.Nk, a.delta, a.H, nqb, sp.nsplit, sp.split_len, rows * D, rows,
                     total, c2, q_sign);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const MergeArgs m{o_parts, l_parts, sp.nsplit, a.o, a.lse, a.B, a.Nq, a.H, a.stream};
  return launch_merge<D>(m);
}

template hipError_t launch_fwd<64, false>(const FwdArgs&);
template hipError_t launch_fwd<64, true>(const FwdArgs&);
template hipError_t launch_fwd<128, false>(const FwdArgs&);
template hipError_t launch_fwd<128, true>(const FwdArgs&);
template hipError_t launch_decode<64, false>(const DecodeArgs&);
template hipError_t launch_decode<64, true>(const DecodeArgs&);
template hipError_t launch_decode<128, false>(const DecodeArgs&);
template hipError_t launch_decode<128, true>(const DecodeArgs&);

}  // namespace fa
