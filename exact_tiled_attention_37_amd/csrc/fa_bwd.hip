// Backward pass of exact tiled attention for gfx950.
//
// The pages require the tiled method's gradients to agree with exact
// attention's within a tolerance (IPLEX post on FlashAttention-2 GPU work
// partitioning, section "Tiling preserves the attention calculation") and
// the method is used to train GPT-style models (FlashAttention-2 abstract on
// the "High-Bandwidth Memory" keyword page); they give no backward equations.
// With loss = sum(dO * O) and P recomputed from the saved logsumexp L:
//   P  = exp(scale * Q K^T - L)         (masked entries are 0)
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D)
//   dQ = scale * dS K,  dK = scale * dS^T Q
// No N x N matrix is stored anywhere: every tile of P and dS exists only in
// registers.
//
// Two kernels on the caller's stream:
//   1. dQ: one workgroup per (block of 128 query rows, head, batch), laid out
//      like the forward pass; each wave owns 32 rows and keeps their Q, dO
//      rows and the dQ accumulator in registers while K/V tiles stream
//      through LDS. Its prologue also forms the row terms of its rows,
//      D = rowsum(dO * O) and L * log2(e), and writes them (D negated) for
//      kernel 2.
//      Per tile:
//        S^T = K Q^T, dP^T = V dO^T        (lane l owns query row l % 32)
//        P^T, dS^T elementwise             (L, D of the lane's own row)
//        dQ^T += K^T dS^T                  (K^T by LDS transpose reads)
//   2. dK/dV: one workgroup per (block of 128 keys, head, batch); each of the
//      4 wavefronts owns 32 keys and keeps their K, V rows and the dK, dV
//      accumulators in registers, while 32-row blocks of Q and dO stream
//      through double-buffered LDS (loaded straight into LDS). Per block:
//        S = Q K^T, dP - D = dO V^T - D    (lane l owns key l % 32; the dP
//                                           accumulators start from -D)
//        P, dS elementwise                 (L, D per row from LDS)
//        dV^T += dO^T P, dK^T += Q^T dS    (dO^T, Q^T by LDS transpose reads)
// Splitting dQ from dK/dV costs two extra products per tile pair (S and dP
// are formed in both kernels) but needs no atomics, no fp32 dQ accumulator in
// memory, no exchange of dS through LDS and no cross-workgroup
// synchronisation, and dQ comes out deterministic.
//
// Rows past the end of the sequence are read as zeros (buffer range check).
// A zero Q or dO row makes that row's terms of dK and dV vanish (its
// recomputed probabilities stay finite: its scores and row terms are 0);
// keys past the end are masked in the dQ kernel's ragged last tile, since a
// probability recomputed from a zero score and a very negative logsumexp can
// overflow. Outputs of such rows are not stored. Causal: only blocks at or
// below the diagonal are visited, waves skip fully masked blocks, only
// diagonal blocks and the ragged end are masked.
// A negative scale is handled by negating the register-resident operand (K
// in dK/dV, Q in dQ) so that the scores keep the caller's sign.

#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kBwdThreads = 256;
constexpr int kKvBlock = 128;  // keys per dK/dV workgroup (4 waves x 32)
constexpr int kQStep = 32;     // query rows per dK/dV step
constexpr int kQBlock = 128;   // query rows per dQ workgroup (4 waves x 32)
constexpr int kKTile = 64;     // keys per dQ tile

// ---------------------------------------------------------------------------
// 2. dK, dV (after the dQ kernel, which writes the row terms it reads).
// BIAS: the bf16 additive bias enters the recomputed probabilities; element
// (b, h, i, j) at Bias[b * bias_sb + h * bias_sh + i * bias_srow + j].
template <int D, bool CAUSAL, bool BIAS = false>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ dsum,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int N, int H, int nkb, int total_blocks,
    float c2, uint32_t k_sign, float dk_scale, const bf16* __restrict__ Bias = nullptr, long bias_sb = 0,
    long bias_sh = 0, int bias_srow = 0) {
  using TQ = Tile<kQStep, D>;    // one Q or dO block (rows = queries)
  using TV = Tile<kKvBlock, D>;  // the workgroup's V rows (rows = keys)
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int QT = TQ::BYTES;
  constexpr int DMA_PER_WAVE = TQ::LOADS / 4;
  __shared__ __attribute__((aligned(1024))) char qbuf[2][2 * QT];  // per stage: Q tile, then dO tile
  __shared__ __attribute__((aligned(256))) float rowbuf[2][2 * 64];  // per stage: L*log2e, then D
  __shared__ __attribute__((aligned(1024))) char vblk[TV::BYTES];
  // Bias of the current step for each wave's 32 keys: 32 query rows x 64
  // bytes, row-major (see bias_dma / the transpose reads in compute).
  __shared__ __attribute__((aligned(1024))) char bias_slice[BIAS ? 4 * kQStep * 64 : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int g = lane >> 5, l32 = lane & 31, G = lane >> 4;

  const HeadRank hr = block_order<CAUSAL>(blockIdx.x, total_blocks / nkb, nkb, 2 * kCusPerXcd, 2);
  const int head = hr.head;
  const int kblk = hr.rank;  // block 0 has the most causal work: it goes first
  const int b = head / H, h = head - b * H;
  const long hoff = ((long)b * N * H + h) * D;
  const uint32_t tokb = (uint32_t)H * D * 2;
  const uint32_t nrec = (uint32_t)(N - 1) * tokb + D * 2;
  const u32x4 rq = make_raw_rsrc(Q + hoff, nrec);
  const u32x4 rdo = make_raw_rsrc(dO + hoff, nrec);
  const u32x4 rl = make_raw_rsrc(lse2 + (long)head * N, (uint32_t)N * 4);
  const u32x4 rd = make_raw_rsrc(dsum + (long)head * N, (uint32_t)N * 4);

  const int kb0 = kblk * kKvBlock;
  const int kw0 = kb0 + 32 * wave;
  const int mykey = kw0 + l32;
  // Bias rows of this (batch, head): N rows of bias_srow elements. Each step
  // the wave's 32 rows x 32 keys (64 bytes per row) go into its LDS slice by
  // two LDS-DMA loads (lane i of load u fills 16-byte slot 64 u + i: row
  // 16 u + i / 4, keys 8 (i % 4) .. + 7 of the wave's 32). The whole offset
  // is per lane, so rows at or past N and keys past the last row's end read
  // as zeros (the library keeps (N + 64) * bias_srow * 2 below 2^32).
  const u32x4 rbr = make_raw_rsrc(BIAS ? Bias + b * bias_sb + h * bias_sh : Q,
                                  BIAS ? (uint32_t)((long)N * bias_srow * 2) : 0u);
  uint32_t bias_dma_off[BIAS ? 2 : 1];
  uint32_t bias_tr_addr = 0;
  const uint32_t bslice_lds = BIAS ? lds_base(bias_slice + wave * kQStep * 64) : 0u;
  if constexpr (BIAS) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      bias_dma_off[u] = ((uint32_t)(16 * u + (lane >> 2)) * (uint32_t)bias_srow +
                         (uint32_t)(kb0 + 32 * wave + 8 * (lane & 3))) * 2u;
    // Transpose reads (ds_read_b64_tr_b16): in each 16-lane group, lane t
    // points at row R + t / 4, keys K0 + 4 (t % 4) .. + 3 (K0 = 16 for the
    // groups holding keys 16..31); lane j then receives key K0 + j of rows
    // R .. R + 3, i.e. its own key's bias for 4 consecutive accumulator rows.
    const int t = lane & 15, k0 = 16 * ((lane >> 4) & 1);
    bias_tr_addr = (uint32_t)((4 * g + (t >> 2)) * 64 + (k0 + 4 * (t & 3)) * 2);
  }
  auto bias_dma = [&](int step) __attribute__((always_inline)) {
    const uint32_t qoff = (uint32_t)(step * kQStep) * (uint32_t)bias_srow * 2u;
#pragma unroll
    for (int u = 0; u < 2; ++u) dma16_at(rbr, bslice_lds + 1024u * u, bias_dma_off[u] + qoff);
  };

  // This wave's K rows as B operands of S = Q K^T (registers), and the
  // block's V rows (LDS, read as B operands of dP = dO V^T).
  bf16x8 kf[KS];
  {
    const auto rk = make_rsrc(K + hoff, nrec);
    const uint32_t koff = row_off(mykey, N, tokb, 16 * g);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rk, koff + 32 * ks) ^ k_sign);
    const u32x4 rv = make_raw_rsrc(V + hoff, nrec);
#pragma unroll
    for (int t = 0; t < TV::LOADS / 4; ++t) {
      const int u = wave + 4 * t;
      const uint32_t off = row_off(kb0 + TV::dma_row(u, lane), N, tokb, 16u * TV::dma_chunk(u, lane));
      dma16(rv, vblk + TV::dma_dst(u), off);
    }
  }

  // A lane's byte offset inside a Q/dO step is a fixed lane part plus a
  // uniform per-load part; the step's position
  // goes into the (scalar) resources, whose ends still turn rows past N into
  // zeros.
  const uint32_t lane_off = TQ::dma_lane_off(lane, tokb);
  const uint32_t qbuf_lds = lds_base(&qbuf[0][0]);
  const uint32_t rows_lds = lds_base(&rowbuf[0][0]);
  auto issue = [&](int step, char* dst, float* rows) __attribute__((always_inline)) {
    const int q0 = step * kQStep;
    const uint32_t toff = (uint32_t)q0 * tokb;
    const u32x4 rqt = rsrc_advance(rq, toff), rdot = rsrc_advance(rdo, toff);
    const uint32_t l0 = qbuf_lds + (uint32_t)(dst - &qbuf[0][0]);
#pragma unroll
    for (int t = 0; t < DMA_PER_WAVE; ++t) {
      const int u = wave + 4 * t;
      const uint32_t off = lane_off + TQ::dma_load_off(u, tokb);
      dma16_at(rqt, l0 + TQ::dma_dst(u), off);
      dma16_at(rdot, l0 + TQ::dma_dst(u) + QT, off);
    }
    if (wave == 0) {  // 64 row terms per load; the 32 past this step are unused
      const u32x4 rlt = rsrc_advance(rl, (uint32_t)q0 * 4), rdt = rsrc_advance(rd, (uint32_t)q0 * 4);
      const uint32_t r0 = rows_lds + (uint32_t)((char*)rows - (char*)&rowbuf[0][0]);
      dma4_at(rlt, r0, (uint32_t)lane * 4);
      dma4_at(rdt, r0 + 64 * 4, (uint32_t)lane * 4);
    }
  };

  f32x16 dvacc[DB], dkacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dvacc[i] = f32x16{};
    dkacc[i] = f32x16{};
  }

  // One step of 32 query rows. MASK: the causal mask is applied (steps that
  // straddle the diagonal); the other steps have no per-element masking.
  const int nqs = (N + kQStep - 1) / kQStep;  // 32-row query steps
  auto compute = [&](int step, const char* qt, const float* rows, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int q0 = step * kQStep;
    const char* dot = qt + QT;
    // Bias of this lane's key for its 16 accumulator rows (queries) from the
    // slice: rows 8 rq + 4 g .. + 3 per transpose read.
    i16x4 bt[BIAS ? 4 : 1];
    if constexpr (BIAS) {
      const char* const bsl = bias_slice + wave * kQStep * 64;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) bt[rq] = lds_read_tr(bsl, (int)bias_tr_addr + 512 * rq);
    }
    // dP starts from -D of the accumulator's rows (the row terms hold -D),
    // so the products leave dP - D in it.
    f32x16 s = f32x16{}, dp;
#pragma unroll
    for (int rq4 = 0; rq4 < 4; ++rq4) {
      const f32x4 nd4 = *reinterpret_cast<const FA_LDS f32x4*>((const FA_LDS float*)rows + 64 + 8 * rq4 + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[4 * rq4 + e] = nd4[e];
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma32(TQ::row8(qt, l32, 2 * ks + g), kf[ks], s);
      dp = mfma32(TQ::row8(dot, l32, 2 * ks + g), TV::row8(vblk, 32 * wave + l32, 2 * ks + g), dp);
    }
    f32x8 p8[2], ds8[2];
#pragma unroll
    for (int rq4 = 0; rq4 < 4; ++rq4) {
      const int qi0 = 8 * rq4 + 4 * g;
      const f32x4 l4 = *reinterpret_cast<const FA_LDS f32x4*>((const FA_LDS float*)rows + qi0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * rq4 + e;
        float p;
        if constexpr (BIAS)
          p = fast_exp2(__builtin_fmaf(
              s[r], c2, __builtin_fmaf(bf16_bits_to_float((uint16_t)bt[rq4][e]), kLog2e, -l4[e])));
        else
          p = fast_exp2(__builtin_fmaf(s[r], c2, -l4[e]));
        if constexpr (MASK) p = (mykey > q0 + qi0 + e) ? 0.f : p;
        p8[r >> 3][r & 7] = p;
        ds8[r >> 3][r & 7] = p * dp[r];
      }
    }
    if constexpr (BIAS) {
      // The slice is read; the next step's bias may overwrite it (the wait
      // orders the LDS-DMA writes after these reads).
      if (step + 1 < nqs) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        bias_dma(step + 1);
      }
    }
    const bf16x8 pb[2] = {to_bf16x8(p8[0]), to_bf16x8(p8[1])};
    const bf16x8 dsb[2] = {to_bf16x8(ds8[0]), to_bf16x8(ds8[1])};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col0 = 32 * db + 16 * (G & 1);
        dvacc[db] = mfma32(TQ::col8(dot, 16 * hh + 4 * g, 16 * hh + 8 + 4 * g, col0, lane), pb[hh], dvacc[db]);
        dkacc[db] = mfma32(TQ::col8(qt, 16 * hh + 4 * g, 16 * hh + 8 + 4 * g, col0, lane), dsb[hh], dkacc[db]);
      }
  };

  // Causal: query blocks start at the diagonal; the first kKvBlock / kQStep
  // of them straddle it and are masked, the rest need no mask. Step s lives
  // in stage (s - s0) % 2; each loop has a single exit, so the accumulators
  // keep their registers across the loop boundaries.
  const int s0 = CAUSAL ? kb0 / kQStep : 0;
  const int sm = CAUSAL ? min(nqs, s0 + kKvBlock / kQStep) : s0;  // masked steps: [s0, sm)
  issue(s0, qbuf[0], rowbuf[0]);
  if constexpr (BIAS) bias_dma(s0);
  wait_vmem();
  __syncthreads();
  int step = s0;
  for (; step < sm; ++step) {
    const int t = (step - s0) & 1;
    if (step + 1 < nqs) issue(step + 1, qbuf[t ^ 1], rowbuf[t ^ 1]);
    // A wave whose keys all follow the step's queries has nothing to add
    // (with a bias the step still runs: it issues the next step's bias).
    if (BIAS || step * kQStep + kQStep - 1 >= kw0) compute(step, qbuf[t], rowbuf[t], std::true_type{});
    wait_vmem();
    __syncthreads();
  }
  for (; step < nqs; ++step) {
    const int t = (step - s0) & 1;
    if (step + 1 < nqs) issue(step + 1, qbuf[t ^ 1], rowbuf[t ^ 1]);
    compute(step, qbuf[t], rowbuf[t], std::false_type{});
    wait_vmem();
    __syncthreads();
  }

  if (mykey < N) {
    bf16* dkrow = dK + hoff + (long)mykey * H * D;
    bf16* dvrow = dV + hoff + (long)mykey * H * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq4 = 0; rq4 < 4; ++rq4) {
        const int d0 = 32 * db + 8 * rq4 + 4 * g;
        const f32x4 k4 = {dkacc[db][4 * rq4] * dk_scale, dkacc[db][4 * rq4 + 1] * dk_scale,
                          dkacc[db][4 * rq4 + 2] * dk_scale, dkacc[db][4 * rq4 + 3] * dk_scale};
        const f32x4 v4 = {dvacc[db][4 * rq4], dvacc[db][4 * rq4 + 1], dvacc[db][4 * rq4 + 2],
                          dvacc[db][4 * rq4 + 3]};
        *reinterpret_cast<bf16x4*>(dkrow + d0) = to_bf16x4(k4);
        *reinterpret_cast<bf16x4*>(dvrow + d0) = to_bf16x4(v4);
      }
  }
}

// ---------------------------------------------------------------------------
// 1. dQ (and the row terms D, L * log2e of every query row).
// BIAS: as in the dK/dV kernel; in addition, when dBias is given, this kernel
// writes dBias = dS (bf16) at dBias[((b * H + h) * N + i) * dbias_srow + j]
// for every query row i < N and key j < N: the tiles it visits write their
// dS (0 where masked), the causal keys it never visits are written as 0.
template <int D, bool CAUSAL, bool BIAS = false>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const bf16* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ lse2, float* __restrict__ dsum,
    bf16* __restrict__ dQ, int N, int H, int nqb, int total_blocks, float c2, uint32_t q_sign,
    float dq_scale, const bf16* __restrict__ Bias = nullptr, long bias_sb = 0, long bias_sh = 0,
    int bias_srow = 0, bf16* __restrict__ dBias = nullptr, int dbias_srow = 0) {
  using T = Tile<kKTile, D>;  // one K or V tile (rows = keys)
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = T::BYTES;
  constexpr int DMA_PER_WAVE = T::LOADS / 4;
  __shared__ __attribute__((aligned(1024))) char kvbuf[2][2 * TILE];  // per stage: K tile, then V tile
  // dBias staging: each wave's 32 rows x 64 keys of dS (see store_dbias).
  constexpr int RB = kKTile * 2;  // bytes per row of a tile's dS
  __shared__ __attribute__((aligned(1024))) char dbias_lds[BIAS ? 4 * 32 * RB : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int g = lane >> 5, l32 = lane & 31, G = lane >> 4;
  char* const dbw_lds = dbias_lds + (BIAS ? wave * 32 * RB : 0);

  const HeadRank hr = block_order<CAUSAL>(blockIdx.x, total_blocks / nqb, nqb, 2 * kCusPerXcd, 2);
  const int head = hr.head;
  const int qblk = nqb - 1 - hr.rank;  // longest causal rows first
  const int b = head / H, h = head - b * H;
  const long hoff = ((long)b * N * H + h) * D;
  const uint32_t tokb = (uint32_t)H * D * 2;
  const uint32_t nrec = (uint32_t)(N - 1) * tokb + D * 2;
  const u32x4 rk = make_raw_rsrc(K + hoff, nrec);
  const u32x4 rv = make_raw_rsrc(V + hoff, nrec);

  const int qw0 = qblk * kQBlock + wave * 32;
  const int myq = qw0 + l32;
  const int key_lim = CAUSAL ? min(myq, N - 1) : N - 1;  // the last key this lane's row sees
  // Bias rows of this (batch, head): N rows of bias_srow elements; a tile's
  // 32 rows x 64 keys per wave go straight into the wave's LDS slice (four
  // whole-wave LDS-DMA loads; lane i fills 16-byte slot 64 t + i, i.e. row
  // s / 8 and chunk (s % 8) ^ (row % 8)). Rows at or past N are clamped to
  // N and keys past a row's end run beyond the resource for the last row:
  // both read as zeros, and keys at or past N are masked anyway.
  const u32x4 rbr = make_raw_rsrc(BIAS ? Bias + b * bias_sb + h * bias_sh : Q,
                                  BIAS ? (uint32_t)((long)N * bias_srow * 2) : 0u);
  uint32_t bias_off[BIAS ? 4 : 1];
  if constexpr (BIAS) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int sl = 64 * t + lane, row = sl >> 3, chunk = (sl & 7) ^ (row & 7);
      bias_off[t] = ((uint32_t)min(qw0 + row, N) * (uint32_t)bias_srow + 8u * chunk) * 2u;
    }
  }
  bf16* const dbrow = (BIAS && dBias) ? dBias + ((long)head * N + myq) * dbias_srow : nullptr;

  // This wave's Q and dO rows as B operands of S^T = K Q^T and dP^T = V dO^T,
  // and the row terms of its rows: D = rowsum(dO * O) (fp32 accumulation of
  // the bf16 products; the two lanes of a row hold half of d each) and
  // L * log2(e), which this kernel also writes for the dK/dV kernel that
  // runs after it. A row that saw no key (possible only with a -inf bias)
  // has L = -inf; +inf here makes every recomputed probability
  // exp2(x - inf) exactly 0.
  bf16x8 qf[KS], dof[KS];
  float l2 = 0.f, dd = 0.f;
  {
    const auto rq = make_rsrc(Q + hoff, nrec);
    const auto rdo = make_rsrc(dO + hoff, nrec);
    const auto ro = make_rsrc(O + hoff, nrec);
    const uint32_t qoff = row_off(myq, N, tokb, 16 * g);
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, qoff + 32 * ks) ^ q_sign);
      dof[ks] = __builtin_bit_cast(bf16x8, buf_load16(rdo, qoff + 32 * ks));
      const bf16x8 of = __builtin_bit_cast(bf16x8, buf_load16(ro, qoff + 32 * ks));
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf((float)of[e], (float)dof[ks][e], dpart);
    }
    const float dsum_row = xhalf_sum(dpart);
    if (myq < N) {
      const long i = (long)head * N + myq;
      const float L = LSE[i];
      l2 = L == -INFINITY ? INFINITY : L * kLog2e;
      dd = dsum_row;
      if (g == 0) {
        lse2[i] = l2;
        dsum[i] = -dd;  // -D: the dK/dV kernel starts its dP accumulators from it
      }
    }
  }

  // A lane's byte offset inside a tile is a fixed lane part plus a uniform
  // per-load part; the tile's position goes into the (scalar) resources,
  // whose ends still turn rows past N into zeros.
  const uint32_t lane_off = T::dma_lane_off(lane, tokb);
  const uint32_t kv_lds = lds_base(&kvbuf[0][0]);
  auto issue = [&](int tile, char* dst) __attribute__((always_inline)) {
    const uint32_t toff = (uint32_t)(tile * kKTile) * tokb;
    const u32x4 rkt = rsrc_advance(rk, toff), rvt = rsrc_advance(rv, toff);
    const uint32_t l0 = kv_lds + (uint32_t)(dst - &kvbuf[0][0]);
#pragma unroll
    for (int t = 0; t < DMA_PER_WAVE; ++t) {
      const int u = wave + 4 * t;
      const uint32_t off = lane_off + T::dma_load_off(u, tokb);
      dma16_at(rkt, l0 + T::dma_dst(u), off);
      dma16_at(rvt, l0 + T::dma_dst(u) + TILE, off);
    }
  };

  f32x16 dqacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dqacc[i] = f32x16{};

  // dBias of a tile from the staging slice, by whole rows: lane i stores
  // 16-byte chunks c = i + 64 t (row c / 8, keys 8 (c % 8) .. + 7), so each
  // store instruction writes 8 full 128-byte row segments. Only rows and
  // keys below N are written. (A wave's LDS operations complete in order,
  // so these reads see this tile's writes and precede the next tile's.)
  auto store_dbias = [&](int key0) __attribute__((always_inline)) {
    if (!dBias) return;
#pragma unroll
    for (int t = 0; t < 32 * RB / 16 / 64; ++t) {
      const int c = lane + 64 * t, row = c >> 3, chunk = c & 7;
      const u32x4 v = lds_read16(dbw_lds, row * RB + ((chunk ^ (row & 7)) << 4));
      const int qrow = qw0 + row, key = key0 + 8 * chunk;
      if (qrow < N) {
        bf16* dst = dBias + ((long)head * N + qrow) * dbias_srow + key;
        if (key + 8 <= N) {
          *reinterpret_cast<u32x4*>(dst) = v;
        } else {
          const bf16x8 v8 = __builtin_bit_cast(bf16x8, v);
          for (int e = 0; key + e < N; ++e) dst[e] = v8[e];
        }
      }
    }
  };

  // The bias of tile j into the slice, issued after the barrier that ends
  // tile j - 1 (whose slice reads are then complete) and before the next K/V
  // tile's loads, so that waiting for it leaves those in flight.
  const uint32_t dbw_lds_addr = lds_base(dbw_lds);
  bool kv_prefetched = false;
  auto bias_issue = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) dma16_at(rbr, dbw_lds_addr + 1024u * t, bias_off[t] + (uint32_t)(j * RB));
  };
  auto bias_wait = [&]() __attribute__((always_inline)) {
    if (kv_prefetched)
      wait_vmem_leave<2 * DMA_PER_WAVE>();
    else
      wait_vmem();
  };

  // One tile of 64 keys, one 32-key half at a time. MASK: causal diagonal.
  auto compute = [&](int j, const char* kt, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int key0 = j * kKTile;
    const char* vt = kt + TILE;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // Without a bias dP^T starts from -D (the lane's row term, a block the
      // compiler keeps outside the loop as the first product's addend), so
      // the products leave dP - D in it; the bias form, short of registers
      // for that block, subtracts D per element.
      f32x16 s = f32x16{}, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = BIAS ? 0.f : -dd;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(T::row8(kt, kb * 32 + l32, 2 * ks + g), qf[ks], s);
        dp = mfma32(T::row8(vt, kb * 32 + l32, 2 * ks + g), dof[ks], dp);
      }
      u32x2 bw[BIAS ? 4 : 1];  // this lane's bias: 4 groups of 4 consecutive keys
      if constexpr (BIAS) {
        if (kb == 0) bias_wait();
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          bw[rg] = *reinterpret_cast<const FA_LDS u32x2*>((const FA_LDS char*)dbw_lds + l32 * RB +
                                                           (((4 * kb + rg) ^ (l32 & 7)) << 4) + 8 * g);
      }
      bf16x8 dsf[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f32x8 x;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          const int r = 8 * hh + s8;
          float p;
          if constexpr (BIAS)
            p = fast_exp2(__builtin_fmaf(s[r], c2, __builtin_fmaf(bf16_elem(bw[r >> 2], r & 3), kLog2e, -l2)));
          else
            p = fast_exp2(__builtin_fmaf(s[r], c2, -l2));
          if constexpr (MASK) {
            // Keys past N are masked explicitly: their K and V rows read as
            // zero, but exp2(0 - L * log2e) overflows to +inf for a row whose
            // logsumexp is below about -88, and inf * 0 in the dQ product
            // would turn the row into NaN (with a bias their bias is row
            // padding as well).
            const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            p = key > key_lim ? 0.f : p;
          }
          x[s8] = p * (BIAS ? dp[r] - dd : dp[r]);
        }
        dsf[hh] = to_bf16x8(x);
      }
      if constexpr (BIAS) {
        // dS of this half into the wave's staging slice in the accumulator
        // layout: row l32, keys 32 kb + 8 rg + 4 g .. + 3 (16-byte chunk
        // 4 kb + rg of the row, slot chunk ^ (row % 8)).
        if (dBias) {
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const u32x4 w = __builtin_bit_cast(u32x4, dsf[rg >> 1]);
            const u32x2 v2 = (rg & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]};
            lds_write8(dbw_lds, l32 * RB + (((4 * kb + rg) ^ (l32 & 7)) << 4) + 8 * g, v2);
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int kr = 32 * kb + 16 * hh;
          const bf16x8 a = T::col8(kt, kr + 4 * g, kr + 8 + 4 * g, 32 * db + 16 * (G & 1), lane);
          dqacc[db] = mfma32(a, dsf[hh], dqacc[db]);
        }
    }
    if constexpr (BIAS) store_dbias(key0);
  };

  // Causal: tiles from jm on straddle the diagonal (masked); earlier tiles
  // need no mask. A ragged last tile (keys past N) runs the masked variant.
  const int kv_len = CAUSAL ? min(N, (qblk + 1) * kQBlock) : N;
  const int ntiles = (kv_len + kKTile - 1) / kKTile;
  const int jm = CAUSAL ? min(qblk * (kQBlock / kKTile), N / kKTile) : N / kKTile;
  // Tile j lives in stage j % 2; single-exit loops as in the dK/dV kernel.
  issue(0, kvbuf[0]);
  wait_vmem();
  __syncthreads();
  int j = 0;
  for (; j < jm; ++j) {
    if constexpr (BIAS) bias_issue(j);
    kv_prefetched = j + 1 < ntiles;
    if (kv_prefetched) issue(j + 1, kvbuf[(j + 1) & 1]);
    compute(j, kvbuf[j & 1], std::false_type{});
    wait_vmem();
    __syncthreads();
  }
  for (; j < ntiles; ++j) {
    if constexpr (BIAS) bias_issue(j);
    kv_prefetched = j + 1 < ntiles;
    if (kv_prefetched) issue(j + 1, kvbuf[(j + 1) & 1]);
    // A tile whose keys all follow this wave's rows adds nothing (with a
    // bias it still runs: it writes the tile's dBias, zeros there).
    if (BIAS || !CAUSAL || j * kKTile <= qw0 + 31) compute(j, kvbuf[j & 1], std::true_type{});
    wait_vmem();
    __syncthreads();
  }

  // Causal: dBias of keys past the visited tiles is 0 (16-byte stores, the
  // two lanes of a row taking alternate 8-key chunks).
  if constexpr (BIAS && CAUSAL) {
    if (dbrow && myq < N) {
      const bf16x8 z = {};
      for (int c = ntiles * (kKTile / 8) + g; 8 * c < N; c += 2) {
        if (8 * c + 8 <= N)
          *reinterpret_cast<bf16x8*>(dbrow + 8 * c) = z;
        else
          for (int e = 0; 8 * c + e < N; ++e) dbrow[8 * c + e] = z[0];
      }
    }
  }

  if (myq < N) {
    bf16* qrow = dQ + hoff + (long)myq * H * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq4 = 0; rq4 < 4; ++rq4) {
        const f32x4 x = {dqacc[db][4 * rq4] * dq_scale, dqacc[db][4 * rq4 + 1] * dq_scale,
                         dqacc[db][4 * rq4 + 2] * dq_scale, dqacc[db][4 * rq4 + 3] * dq_scale};
        *reinterpret_cast<bf16x4*>(qrow + 32 * db + 8 * rq4 + 4 * g) = to_bf16x4(x);
      }
  }
}

}  // namespace

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdArgs& a) {
  const float c2 = fabsf(a.scale) * kLog2e;
  const uint32_t sign = a.scale < 0.f ? 0x80008000u : 0u;
  {  // dQ first: it also writes the row terms (L * log2e, D) the dK/dV kernel reads
    const int nqb = (a.N + kQBlock - 1) / kQBlock;
    const int total = a.B * a.H * nqb;
    if (a.bias)
      hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, true>), dim3(total), dim3(kBwdThreads), 0, a.stream,
                         static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                         static_cast<const bf16*>(a.v), static_cast<const bf16*>(a.dout),
                         static_cast<const bf16*>(a.o), a.lse, a.lse2, a.dsum, static_cast<bf16*>(a.dq), a.N,
                         a.H, nqb, total, c2, sign, a.scale, static_cast<const bf16*>(a.bias), a.bias_sb,
                         a.bias_sh, a.bias_srow, static_cast<bf16*>(a.dbias), a.dbias_srow);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(total), dim3(kBwdThreads), 0, a.stream,
                         static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                         static_cast<const bf16*>(a.v), static_cast<const bf16*>(a.dout),
                         static_cast<const bf16*>(a.o), a.lse, a.lse2, a.dsum, static_cast<bf16*>(a.dq), a.N,
                         a.H, nqb, total, c2, sign, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nkb = (a.N + kKvBlock - 1) / kKvBlock;
    const int total = a.B * a.H * nkb;
    if (a.bias)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, true>), dim3(total), dim3(kBwdThreads), 0, a.stream,
                         static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                         static_cast<const bf16*>(a.v), static_cast<const bf16*>(a.dout), a.lse2,
                         a.dsum, static_cast<bf16*>(a.dk), static_cast<bf16*>(a.dv), a.N, a.H, nkb,
                         total, c2, sign, a.scale, static_cast<const bf16*>(a.bias), a.bias_sb, a.bias_sh,
                         a.bias_srow);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(total), dim3(kBwdThreads), 0, a.stream,
                         static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                         static_cast<const bf16*>(a.v), static_cast<const bf16*>(a.dout), a.lse2,
                         a.dsum, static_cast<bf16*>(a.dk), static_cast<bf16*>(a.dv), a.N, a.H, nkb,
                         total, c2, sign, a.scale);
    return hipGetLastError();
  }
}

template hipError_t launch_bwd<64, false>(const BwdArgs&);
template hipError_t launch_bwd<64, true>(const BwdArgs&);
template hipError_t launch_bwd<128, false>(const BwdArgs&);
template hipError_t launch_bwd<128, true>(const BwdArgs&);

}  // namespace fa
