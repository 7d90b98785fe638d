// FP8 (e4m3) forward of exact tiled attention for gfx950.
//
// Low-precision attention (an abstract on the related-papers page for
// "FlashAttention on a Napkin" runs attention on narrow-format matrix units)
// moved to the MI355X FP8 matrix unit: Q, K and V arrive as OCP E4M3 codes
// with one float32 descale per (batch, head) and tensor, and both products run
// on v_mfma_scale_f32_32x32x64_f8f6f4 (64-deep, twice the bf16 rate). The
// tiling, online softmax, deferred normalisation and causal skipping are
// those of the bf16 forward (IPLEX post on FlashAttention-2 work
// partitioning, sections "Tiling preserves the attention calculation" and
// "Three changes improve GPU utilisation").
//
// What changes with 8-bit operands:
//   * S^T = K Q^T: a lane's A/B operand is 32 consecutive bytes of a K or Q
//     row (both operands use the same byte order, so the reduction pairs
//     them correctly); the descales of Q and K fold into the exp2 scale.
//   * P is rounded to e4m3 for the PV product. It is taken as
//     2^4 * exp2(s - m) with the running max m allowed to lag as long as
//     every value stays <= 448 (the largest e4m3 number), so values down
//     to 2^-10 of the row maximum still land on normal e4m3 numbers. The row sum uses the fp32
//     values; the scale cancels in O = (P V) / l and is removed from the
//     logsumexp.
//   * P^T comes straight from the S^T accumulators: with the V rows of a
//     tile stored in LDS in a key order that exchanges bits 2 and 3 of the
//     key index, byte p of a lane's P operand (accumulator p % 16 of 32-key
//     block p / 16) meets byte p of its V^T operand, which four 8-bit
//     transpose loads (ds_read_b64_tr_b8) deliver.
//   * LDS tiles hold 64 rows of 128 bytes (d = 128); the 16-byte chunk c of
//     row r sits at position c ^ h(r), h(r) = 2 ((r / 2) % 4) + (r / 8) % 2.
//     A row fills half of the 256 bytes the 64 banks serve per pass, so the
//     16 rows one row read touches (16 lanes, same chunk) must spread over
//     both halves and 8 positions: rows of equal parity need distinct h
//     within 16 rows. The transpose reads of V (32 lanes: chunks c and c ^ 1
//     of 8 consecutive rows) need distinct h / 2 among the 4 rows of equal
//     parity within 8. This h gives both; h = r % 8 (rows r and r + 8 alike)
//     made every K row read a two-way conflict.
// O is written as bf16 (times the V descale), the logsumexp as fp32.
//
// Microscaled form (MX): instead of the per-head descales, one E8M0 scale
// (2^(code - 127)) per 32 consecutive elements along each product's
// reduction dimension, applied by the matrix instruction itself through its
// per-lane scale operands. The instruction pairs a lane's scale with one
// 32-deep block of its 64-deep reduction: bytes 0-15 of lanes m and m + 32
// form block 0 (the scale of lane m), bytes 16-31 of both form block 1 (the
// scale of lane m + 32). So in this form, with KS = d / 64 k-steps, lane
// half g loads d = 32 ks + 16 g .. + 15 into bytes 0-15 and d = 32 (KS +
// ks) + 16 g .. + 15 into bytes 16-31 of the Q and K operands: block 0 of
// k-step ks is d-block ks, block 1 is d-block KS + ks, and lane half g needs
// d-blocks KS g .. KS g + KS - 1 (consecutive bytes of a token's d / 32
// scale bytes: one 16-bit read at d = 128, one byte at d = 64). The P and
// V^T operands already hold key block g of the tile in that position (key
// rows 8 g .. + 7 and 16 + 8 g .. + 7 of each 32-key block, the V^T
// transpose reads above), so V's scale for (column, 32-key block) is lane
// (column, g)'s. At d = 128 each tile's K and V scales come into LDS with
// the tile (one 4-byte LDS-DMA per lane and tensor); at d = 64 (2 bytes per
// token, which a 4-byte load would read past a sequence's last token) each
// lane loads its own into registers a tile ahead. Q's stay in a register.
// P's scale is 2^0.

#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kF8BR = 128;                 // query rows per workgroup (4 waves x 32)
constexpr int kF8BC = 64;                  // keys per K/V tile
constexpr int kF8Threads = 256;
constexpr float kF8PMax = 448.f;           // largest finite e4m3 value
constexpr float kF8NoMax = -1e30f;         // running max of a row that has seen no key
constexpr float kF8Shift = 4.f;            // P is scaled by 2^4 before rounding

// Position of 16-byte chunk c of row r in an LDS tile of D-byte rows (D = the
// head dimension): c ^ h(r). d = 128 above; d = 64 (four rows per 256-byte
// bank pass): rows of equal r % 4 among 16 consecutive rows need distinct h
// (K row reads), and rows r and r + 4 need h differing in bit 1 (the V
// transpose reads take chunks 2 db and 2 db + 1 of 8 consecutive rows):
// h(r) = 2 ((r / 4) % 2) + (r / 8) % 2.
template <int D>
__device__ __forceinline__ constexpr int f8_swz(int r) {
  if constexpr (D == 128)
    return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
  else
    return (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
}
template <int D>
__device__ __forceinline__ constexpr int f8_slot(int r, int c) { return r * D + ((c ^ f8_swz<D>(r)) << 4); }
// LDS row r of a V tile holds key row vperm(r) (bits 2 and 3 exchanged; an involution).
__device__ __forceinline__ constexpr int vperm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);  // scales 2^0
}

__device__ __forceinline__ i32x2 lds_read_tr8(const char* base, int off) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2*)((FA_LDS char*)base + off));
}

__device__ __forceinline__ i32x8 cat(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// d = 128: three workgroups per CU (3 waves per SIMD, 168 registers, 96 KiB
// of LDS): with the matrix time halved, a third wave hides more of the
// softmax. d = 64 fits four (128 registers, 16 KiB of LDS each; measured
// 2-15% faster than three). MX: block scales (q_scale, k_scale, v_scale)
// instead of the descales.
template <int D>
constexpr int kF8Waves = D == 64 ? 4 : 3;
template <int D, bool CAUSAL, bool MX>
__global__ __launch_bounds__(kF8Threads) __attribute__((amdgpu_waves_per_eu(kF8Waves<D>, kF8Waves<D>))) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ q_descale, const float* __restrict__ k_descale, const float* __restrict__ v_descale,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int H, int nqb, int total_blocks, float scale,
    const uint8_t* __restrict__ q_scale, const uint8_t* __restrict__ k_scale, const uint8_t* __restrict__ v_scale) {
  constexpr int KS = D / 64;        // 64-deep k-steps of S over d
  constexpr int DB = D / 32;        // 32-column blocks of the output
  constexpr int CH = D / 16;        // 16-byte chunks per row
  constexpr int TILE = kF8BC * D;   // bytes of one K or V tile
  constexpr int RPL = 1024 / D;     // rows per whole-wave 1 KiB load
  constexpr int LPW = D / 64;       // such loads per wave, tensor and tile
  // MX at d = 128: the tile's scales go through LDS (below); at d = 64 a
  // token's two scale bytes are read straight into registers.
  constexpr bool SLDS = MX && D == 128;
  __shared__ __attribute__((aligned(1024))) char ring[2][2 * TILE];  // per stage: K tile, V tile
  // MX (d = 128), per stage: the tile's K scales (64 keys x 4 blocks of d),
  // then its V scales (2 key blocks x 128 columns).
  __shared__ __attribute__((aligned(256))) char scl[SLDS ? 2 : 1][SLDS ? 512 : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, G = lane >> 4, j16 = lane & 15;

  const HeadRank hr = block_order<CAUSAL>(blockIdx.x, total_blocks / nqb, nqb, kF8Waves<D> * kCusPerXcd, 2);
  const int head = hr.head;                            // b * H + h
  const int qblk = nqb - 1 - hr.rank;                  // longest causal rows first
  const int b = head / H, h = head - b * H;
  const float qk = MX ? scale : scale * q_descale[head] * k_descale[head];
  const float c2 = fabsf(qk) * kLog2e;
  const uint32_t q_sign = qk < 0.f ? 0x80808080u : 0u;  // a negative factor negates Q
  const float v_mul = MX ? 1.f : v_descale[head];
  const long hoff = ((long)b * N * H + h) * D;         // byte offset of token 0
  const uint32_t tokb = (uint32_t)H * D;
  const uint32_t nrec = (uint32_t)(N - 1) * tokb + D;
  const auto rq = make_rsrc(Q + hoff, nrec);
  const u32x4 rk = make_raw_rsrc(K + hoff, nrec);
  const u32x4 rv = make_raw_rsrc(V + hoff, nrec);

  const int qw0 = qblk * kF8BR + wave * 32;
  const int myq = qw0 + l32;
  const int key_lim = CAUSAL ? min(myq, N - 1) : N - 1;  // the last key this lane's row sees

  // Q as the B operand: bytes 64 ks + 32 g .. +31 of row myq (MX: bytes
  // 32 ks + 16 g .. + 15 and 32 (KS + ks) + 16 g .. + 15, see above).
  i32x8 qf[KS];
  {
    const uint32_t qoff = row_off(myq, N, tokb, (MX ? 16u : 32u) * g);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 lo = buf_load16(rq, qoff + (MX ? 32 : 64) * ks) ^ q_sign;
      const u32x4 hi = buf_load16(rq, qoff + (MX ? 32 * (KS + ks) : 64 * ks + 16)) ^ q_sign;
      qf[ks] = cat(lo, hi);
    }
  }
  // MX: Q's scales of row myq (D / 32 bytes, d-block i in byte i), shifted so
  // that this lane half's block of k-step ks (KS g + ks) is byte ks. Block
  // scales of a tile's keys and values: rows and key blocks past the end read
  // as zeros. At d = 128 they come from wave 0 (K: lane i, the 4 bytes of key
  // row i) and wave 1 (V: lane i, bytes 4 (i % 32) .. + 3 of key block
  // i / 32), the tile's position in the (scalar) resource and the lane's
  // part fixed.
  uint32_t qsw = 0;
  u32x4 rks = {}, rvs = {};
  constexpr int SB = D / 32;                               // scale bytes per token of q_scale / k_scale
  const uint32_t srow = (uint32_t)H * SB;                  // bytes between tokens of q_scale / k_scale
  const uint32_t vrow = (uint32_t)H * D;                   // bytes between key blocks of v_scale
  const int nvb = (N + 31) / 32;
  if constexpr (MX) {
    const long sbase = ((long)b * N * H + h) * SB;
    const auto rqs = make_rsrc(q_scale + sbase, (uint32_t)(N - 1) * srow + SB);
    const int qsoff = (int)((uint32_t)min(myq, N) * srow);
    if constexpr (D == 128)
      qsw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rqs, qsoff, 0, 0) >> (16 * g);
    else
      qsw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rqs, qsoff, 0, 0) >> (8 * g);
    rks = make_raw_rsrc(k_scale + sbase, (uint32_t)(N - 1) * srow + SB);
    rvs = make_raw_rsrc(v_scale + ((long)b * nvb * H + h) * D, (uint32_t)(nvb - 1) * vrow + D);
  }
  // MX at d = 64: the next tile's scales, loaded into registers one tile
  // ahead: K's two bytes of this lane's key row in each 32-key block, V's
  // byte of column 32 db + l32 in key block g.
  uint32_t ksn[2] = {0u, 0u}, vsn[2] = {0u, 0u}, ksc[2] = {0u, 0u}, vsv[2] = {0u, 0u};
  const uint8_t* const ksb = MX ? k_scale + ((long)b * N * H + h) * SB : nullptr;
  const uint8_t* const vsb = MX ? v_scale + ((long)b * nvb * H + h) * D : nullptr;
  auto scale_loads = [&](int tile) __attribute__((always_inline)) {
    if constexpr (MX && D == 64) {
      // (the tile starts below N: both offsets stay inside the records)
      const uint32_t ko = (uint32_t)tile * (kF8BC * srow), vo = (uint32_t)tile * (2 * vrow);
      const auto rk2 = make_rsrc(ksb + ko, (uint32_t)(N - 1) * srow + SB - ko);
      const auto rv2 = make_rsrc(vsb + vo, (uint32_t)(nvb - 1) * vrow + D - vo);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) ksn[kb] = buf_load2(rk2, (uint32_t)(32 * kb + l32) * srow);
#pragma unroll
      for (int db = 0; db < 2; ++db)
        vsn[db] = (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(rv2, (int)((uint32_t)g * vrow + 32u * db + l32), 0, 0);
    }
  };

  // LDS-DMA of one tile: wave load u fills LDS rows RPL u .. RPL u + RPL - 1
  // (d = 128: 8 rows of 8 chunks; d = 64: 16 rows of 4 chunks); lane i
  // writes slot i, i.e. row RPL u + i / CH at chunk position i % CH.
  auto issue = [&](int tile, char* dst, char* sdst) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < LPW; ++t) {
      const int u = wave + 4 * t;
      const int r = RPL * u + lane / CH;
      const uint32_t c16 = 16u * (uint32_t)((lane % CH) ^ f8_swz<D>(r));
      dma16(rk, dst + u * 1024, row_off(tile * kF8BC + r, N, tokb, c16));
      dma16(rv, dst + TILE + u * 1024, row_off(tile * kF8BC + vperm(r), N, tokb, c16));
    }
    if constexpr (SLDS) {
      // (The tile starts below N, so the advanced resource keeps a positive
      // record count: rows and key blocks past the end read as zeros.)
      if (wave == 0)
        dma4(rsrc_advance(rks, (uint32_t)tile * (kF8BC * srow)), sdst, (uint32_t)lane * srow);
      else if (wave == 1)
        dma4(rsrc_advance(rvs, (uint32_t)tile * (2 * vrow)), sdst + 256, (uint32_t)(lane >> 5) * vrow + 4u * (lane & 31));
    }
  };

  const int kv_len = CAUSAL ? min(N, (qblk + 1) * kF8BR) : N;
  const int ntiles = (kv_len + kF8BC - 1) / kF8BC;

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = kF8NoMax;
  float l_run = 0.f;

  // Per-lane LDS offsets: K row reads (row l32 of a 32-key block, chunk
  // 4 ks + 2 g + hi; MX: 2 (hi KS + ks) + g) and V transpose reads (row 8 g + j16 / 2 of a 16-key
  // group, chunk 2 db + G % 2, byte half j16 % 2); the block and group add
  // whole rows, which leave the swizzle unchanged (it reads row bits 1-3).
  int koff[KS][2], voff[DB];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) koff[ks][hi] = f8_slot<D>(l32, MX ? 2 * (hi * KS + ks) + g : 4 * ks + 2 * g + hi);
#pragma unroll
  for (int db = 0; db < DB; ++db) voff[db] = f8_slot<D>(8 * g + (j16 >> 1), 2 * db + (G & 1)) + 8 * (j16 & 1);

  i32x8 pf = {};  // P^T operand of the current tile (kept across tiles)
  auto scores = [&](f32x16 (&s)[2], const char* kt, const char* st, int key0, auto mask_tag)
                    __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    s[0] = f32x16{};
    s[1] = f32x16{};
    uint32_t ksw[2] = {0u, 0u};  // MX: this lane half's K scales of its key row in block kb, as qsw
    if constexpr (SLDS) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        ksw[kb] = *reinterpret_cast<const FA_LDS uint16_t*>((const FA_LDS char*)st + (32 * kb + l32) * 4 + 2 * g);
    } else if constexpr (MX) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) ksw[kb] = ksc[kb] >> (8 * g);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const i32x8 a = cat(lds_read16(kt, koff[ks][0] + kb * 32 * D), lds_read16(kt, koff[ks][1] + kb * 32 * D));
        if constexpr (MX) {
          if (ks == 0)
            s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], s[kb], 0, 0, 0, (int)ksw[kb], 0, (int)qsw);
          else
            s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], s[kb], 0, 0, 1, (int)ksw[kb], 1, (int)qsw);
        } else {
          s[kb] = mfma_f8(a, qf[ks], s[kb]);
        }
      }
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key > key_lim) s[kb][r] = -INFINITY;
        }
    }
  };
  // The P^T operand (byte p = 2^4 * exp2(s - m) of accumulator p % 16 of
  // block p / 16) from the scores and bias = 2^4 / m in log2 units; returns
  // this lane's fp32 sum of the tile's P and, in gmax, the largest sum of
  // one of its groups of four values.
  auto probs = [&](const f32x16 (&s)[2], float bias, auto mask_tag, float& gmax) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    float t = 0.f;
    gmax = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sv = s[w >> 2][4 * (w & 3) + i];
        float x = fast_exp2(__builtin_fmaf(sv, c2, bias));
        if constexpr (MASK) x = (sv == -INFINITY) ? 0.f : x;
        e[i] = x;
      }
      const float ws = (e[0] + e[1]) + (e[2] + e[3]);
      t += ws;
      gmax = vmax(gmax, ws);
      // The two conversions write the low and the high half of the word; the
      // other half starts as the previous tile's value (no zeroing move).
      int d = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], pf[w], false);
      pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], d, true);
    }
    return t;
  };
  // As in the bf16 forward, the running max only moves when a value of P
  // would leave e4m3's range: P is first taken from the current running max,
  // and it stands if every group of four values of every lane sums to at
  // most 448 (then every value is at most 448, the largest e4m3 number; with
  // the running max at the row maximum a group sums to at most 4 * 2^4).
  // Otherwise (and on the first tile) the scores are formed again, the row
  // maxima taken, O and l rescaled and P recomputed. A row that has seen no
  // key holds the finite kF8NoMax, for which every visible score overflows
  // to +inf and takes that path.
  auto compute = [&](int j, const char* kt, const char* st, auto mask_tag, bool first) __attribute__((always_inline)) {
    const int key0 = j * kF8BC;
    const char* vt = kt + TILE;
    f32x16 s[2];
    scores(s, kt, st, key0, mask_tag);
    float t = 0.f;
    bool slow = true;  // wave-uniform
    if (!first) {
      float gmax;
      t = probs(s, kF8Shift - m_run, mask_tag, gmax);
      slow = __builtin_amdgcn_ballot_w64(!(gmax <= kF8PMax)) != 0;
    }
    if (slow) {
      asm volatile("" ::: "memory");  // a branch; the scores below are loaded again
      if (!first) scores(s, kt, st, key0, mask_tag);
      float mx = max16(s[1], max16(s[0], -INFINITY));
      mx = xhalf_max(mx);
      const float tile_m = (mx == -INFINITY) ? -INFINITY : mx * c2;
      const bool grow = tile_m > m_run;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        asm volatile("" ::: "memory");
        const float m_new = grow ? tile_m : m_run;
        const float alpha = fast_exp2(m_run - m_new);  // 0 from kF8NoMax, 1 when unchanged
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        m_run = m_new;
      }
      float gmax;
      t = probs(s, kF8Shift - m_run, mask_tag, gmax);
    }
    l_run += t;
    // O^T += V^T P^T: for each 32-column block of d, four transpose loads.
    // MX: V's scales of columns 32 db + l32 in key block g of the tile (read
    // together ahead of the products); P's scale is 2^0.
    uint32_t vsc[MX ? DB : 1];
    if constexpr (SLDS) {
#pragma unroll
      for (int db = 0; db < DB; ++db) vsc[db] = *((const FA_LDS uint8_t*)st + 256 + 128 * g + 32 * db + l32);
    } else if constexpr (MX) {
#pragma unroll
      for (int db = 0; db < DB; ++db) vsc[db] = vsv[db];
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      i32x8 a;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const i32x2 t = lds_read_tr8(vt, voff[db] + 16 * q4 * D);
        a[2 * q4] = t[0];
        a[2 * q4 + 1] = t[1];
      }
      if constexpr (MX) {
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf, oacc[db], 0, 0, 0, (int)vsc[db], 0, 127);
      } else {
        oacc[db] = mfma_f8(a, pf, oacc[db]);
      }
    }
  };

  const int jm = CAUSAL ? min(qblk * (kF8BR / kF8BC), N / kF8BC) : N / kF8BC;
  auto sstage = [&](int j) __attribute__((always_inline)) { return scl[SLDS ? (j & 1) : 0]; };
  // MX at d = 64: the next tile's loads (ksn, vsn) become the current
  // tile's scales (ksc, vsv) after each tile's wait.
  auto rotate = [&]() __attribute__((always_inline)) {
    if constexpr (MX && D == 64) {
      ksc[0] = ksn[0];
      ksc[1] = ksn[1];
      vsv[0] = vsn[0];
      vsv[1] = vsn[1];
    }
  };
  issue(0, ring[0], sstage(0));
  scale_loads(0);
  wait_vmem();
  rotate();
  __syncthreads();
  int j = 0;
  for (; j < jm; ++j) {
    if (j + 1 < ntiles) {
      issue(j + 1, ring[(j + 1) & 1], sstage(j + 1));
      scale_loads(j + 1);
    }
    compute(j, ring[j & 1], sstage(j), std::false_type{}, j == 0);
    wait_vmem();
    rotate();
    __syncthreads();
  }
  for (; j < ntiles; ++j) {
    if (j + 1 < ntiles) {
      issue(j + 1, ring[(j + 1) & 1], sstage(j + 1));
      scale_loads(j + 1);
    }
    // (Non-causal: always true here; as a branch it keeps the register
    // allocator from spilling around the masked tile, which it does when
    // the call is unconditional.)
    if (j * kF8BC <= (CAUSAL ? qw0 + 31 : N - 1)) compute(j, ring[j & 1], sstage(j), std::true_type{}, j == 0);
    wait_vmem();
    rotate();
    __syncthreads();
  }

  const float l_tot = xhalf_sum(l_run);
  const bool seen = l_tot > 0.f;
  const float inv = seen ? v_mul / l_tot : 0.f;
  if (myq < N) {
    if (g == 0) LSE[(long)head * N + myq] = seen ? (m_run - kF8Shift + log2f(l_tot)) * kLn2 : -INFINITY;
    bf16* orow = O + ((long)b * N * H + h) * D + (long)myq * H * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq4 = 0; rq4 < 4; ++rq4) {
        const f32x4 x = {oacc[db][4 * rq4] * inv, oacc[db][4 * rq4 + 1] * inv, oacc[db][4 * rq4 + 2] * inv,
                         oacc[db][4 * rq4 + 3] * inv};
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * rq4 + 4 * g) = to_bf16x4(x);
      }
  }
}

}  // namespace

template <bool CAUSAL>
hipError_t launch_fwd_fp8(const Fp8Args& a) {
  const int nqb = (a.N + kF8BR - 1) / kF8BR;
  const int total = a.B * a.H * nqb;
  auto go = [&](auto dtag, auto mxtag) {
    constexpr int D = decltype(dtag)::value;
    constexpr bool MX = decltype(mxtag)::value;
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, MX>), dim3(total), dim3(kF8Threads), 0, a.stream,
                       static_cast<const uint8_t*>(a.q), static_cast<const uint8_t*>(a.k),
                       static_cast<const uint8_t*>(a.v), a.q_descale, a.k_descale, a.v_descale,
                       static_cast<bf16*>(a.o), a.lse, a.N, a.H, nqb, total, a.scale, a.q_scale, a.k_scale,
                       a.v_scale);
  };
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (a.d == 64)
    a.q_scale ? go(D64{}, std::true_type{}) : go(D64{}, std::false_type{});
  else
    a.q_scale ? go(D128{}, std::true_type{}) : go(D128{}, std::false_type{});
  return hipGetLastError();
}

template hipError_t launch_fwd_fp8<false>(const Fp8Args&);
template hipError_t launch_fwd_fp8<true>(const Fp8Args&);

}  // namespace fa
