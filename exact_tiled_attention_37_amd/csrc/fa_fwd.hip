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
// Two (d = 128) or three (d = 64) workgroups share a CU, so one wave's
// softmax arithmetic overlaps another's matrix instructions.
//
// K/V tiles move from memory straight into LDS with buffer loads
// that write LDS directly (no register staging), double-buffered: the next
// tile streams in while the current one is used. Rows past the end of the
// sequence come back as zeros from the buffer range check.
//
// Per wave and K/V tile (64 keys at d = 128, 32 at d = 64):
//   S^T = K Q^T     (MFMA; lane l owns query row l % 32, so a row's scores
//                    sit in two lanes: l and l ^ 32)
//   online softmax in the log2 domain: c2 = |scale| * log2(e) is folded into
//   one FMA per score before exp2; the row max needs a single cross-half
//   exchange; the running sum stays per lane until the epilogue; the
//   division by the row sum is deferred to the epilogue; and the running
//   max (with the rescale of the partial output) is only moved when a row's
//   max grows by more than 2^8, which keeps every exponent <= 8 while
//   skipping almost all rescales.
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

constexpr int kFwdBR = 128;     // query rows per workgroup
constexpr int kFwdThreads = 256;

// Per head dimension: keys per K/V tile and waves per SIMD. d = 64 uses
// 32-key tiles so that three workgroups fit per CU (fewer registers and LDS
// per workgroup); d = 128 uses 64-key tiles at two workgroups per CU.
template <int D> struct FwdCfg;
template <> struct FwdCfg<64> { static constexpr int BC = 32, WAVES_PER_SIMD = 3; };
template <> struct FwdCfg<128> { static constexpr int BC = 64, WAVES_PER_SIMD = 2; };
constexpr float kRescaleSlack = 8.f;  // log2 units a row max may exceed the running max

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads)
__attribute__((amdgpu_waves_per_eu(FwdCfg<D>::WAVES_PER_SIMD, FwdCfg<D>::WAVES_PER_SIMD))) void fwd_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int H, int nqb, int total_blocks,
    float c2, uint32_t q_sign) {
  constexpr int kFwdBC = FwdCfg<D>::BC;            // keys per K/V tile
  constexpr int KB = kFwdBC / 32;                  // 32-key score blocks per tile
  using T = Tile<kFwdBC, D>;                       // one K or V tile in LDS
  constexpr int TILE = T::BYTES;
  constexpr int DMA_PER_WAVE = T::LOADS / 4;       // 1 KiB wave loads per tile per wave
  constexpr int KS = D / 16;                       // MFMA k-steps over d
  constexpr int DB = D / 32;                       // 32-wide output column blocks
  __shared__ __attribute__((aligned(1024))) char kv0[2 * TILE];  // K tile, then V tile
  __shared__ __attribute__((aligned(1024))) char kv1[2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, G = lane >> 4;

  const int logical = xcd_remap(blockIdx.x, total_blocks);
  const int head = logical / nqb;                  // b * H + h
  const int qblk = nqb - 1 - (logical - head * nqb);  // longest causal rows first
  const int b = head / H, h = head - b * H;
  const long hoff = ((long)b * N * H + h) * D;     // element offset of token 0
  const uint32_t tokb = (uint32_t)H * D * 2;       // bytes between tokens
  const uint32_t nrec = (uint32_t)(N - 1) * tokb + D * 2;
  const auto rq = make_rsrc(Q + hoff, nrec);
  const auto rk = make_rsrc(K + hoff, nrec);
  const auto rv = make_rsrc(V + hoff, nrec);

  const int qw0 = qblk * kFwdBR + wave * 32;       // first query row of this wave
  const int myq = qw0 + l32;

  // Q as the B operand of S^T = K Q^T: row myq, d = 16*ks + 8*g .. +7.
  bf16x8 qf[KS];
  {
    const uint32_t qoff = row_off(myq, N, tokb, 16 * g);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, qoff + 32 * ks) ^ q_sign);
  }

  // LDS-DMA: wave load u = wave + 4 t of a tile; lane i fills the chunk
  // (row, column) the layout assigns to it. A tile row is a key.
  auto issue = [&](int tile, char* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < DMA_PER_WAVE; ++t) {
      const int u = wave + 4 * t;
      const uint32_t off = row_off(tile * kFwdBC + T::dma_row(u, lane), N, tokb, 16u * T::dma_chunk(u, lane));
      char* l = dst + T::dma_dst(u);
      buf_load16_lds(rk, l, off);
      buf_load16_lds(rv, l + TILE, off);
    }
  };

  const int kv_len = CAUSAL ? min(N, (qblk + 1) * kFwdBR) : N;
  const int ntiles = (kv_len + kFwdBC - 1) / kFwdBC;

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running max of c2 * score (log2 domain), possibly stale by <= 8
  float l_run = 0.f;        // this lane's share of the running sum

  // One K/V tile. MASK selects the variant for tiles that straddle the
  // causal diagonal or the end of the sequence; all other tiles run the
  // variant without any per-element masking.
  auto compute = [&](int j, const char* kt, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int key0 = j * kFwdBC;
    const char* vt = kt + TILE;
    // The KB accumulation chains are interleaved (independent MFMAs back to back).
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = mfma32(T::row8(kt, kb * 32 + l32, 2 * ks + g), qf[ks], s[kb]);
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if ((CAUSAL && key > myq) || key >= N) s[kb][r] = -INFINITY;
        }
    }
    float mx = max16(s[0], -INFINITY);
#pragma unroll
    for (int kb = 1; kb < KB; ++kb) mx = max16(s[kb], mx);
    mx = xhalf_max(mx);
    const float tile_m = (mx == -INFINITY) ? -INFINITY : mx * c2;
    const bool grow = tile_m > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {  // wave-uniform, rarely taken
      asm volatile("" ::: "memory");          // keep it a branch (no speculation)
      const float m_new = grow ? tile_m : m_run;
      // 0 when m_run = -inf, 1 when unchanged (and when no key was visible yet)
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

    // P in bf16 for the PV product; the row sum stays in fp32 (the
    // logsumexp is checked against the exact value, so it must not inherit
    // the bf16 rounding of P).
    bf16x8 pf[2 * KB];
#pragma unroll
    for (int ks = 0; ks < 2 * KB; ++ks) {
      f32x8 p;
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) {
        const float sv = s[ks >> 1][8 * (ks & 1) + s8];
        float e = fast_exp2(__builtin_fmaf(sv, c2, -m_use));
        if constexpr (MASK) e = (sv == -INFINITY) ? 0.f : e;  // exact zero even when c2 = 0
        p[s8] = e;
      }
      l_run += sum8(p);
      pf[ks] = to_bf16x8(p);
    }
#pragma unroll
    for (int ks = 0; ks < 2 * KB; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 a = T::col8(vt, 16 * ks + 4 * g, 16 * ks + 8 + 4 * g, 32 * db + 16 * (G & 1), lane);
        oacc[db] = mfma32(a, pf[ks], oacc[db]);
      }
  };
  // Tiles before jm need no mask for any wave of this workgroup; they run in
  // a loop of their own so that the masked variant never joins the hot loop.
  // Both loops go through the tiles in pairs so that each LDS buffer is named
  // statically (tile j lives in buffer j % 2).
  const int jm = CAUSAL ? min(qblk * (kFwdBR / kFwdBC), N / kFwdBC) : N / kFwdBC;
  issue(0, kv0);
  wait_vmem();
  __syncthreads();
  int j = 0;
  for (; j + 1 < jm; j += 2) {
    issue(j + 1, kv1);
    compute(j, kv0, std::false_type{});
    wait_vmem();
    __syncthreads();
    if (j + 2 < ntiles) issue(j + 2, kv0);
    compute(j + 1, kv1, std::false_type{});
    wait_vmem();
    __syncthreads();
  }
  for (; j < ntiles; j += 2) {
    if (j + 1 < ntiles) issue(j + 1, kv1);
    compute(j, kv0, std::true_type{});
    wait_vmem();
    __syncthreads();
    if (j + 1 >= ntiles) break;
    if (j + 2 < ntiles) issue(j + 2, kv0);
    compute(j + 1, kv1, std::true_type{});
    wait_vmem();
    __syncthreads();
  }

  const float l_tot = xhalf_sum(l_run);
  const float inv = 1.f / l_tot;
  if (myq < N) {
    if (g == 0) LSE[(long)head * N + myq] = (m_run + log2f(l_tot)) * kLn2;
    bf16* orow = O + hoff + (long)myq * H * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq4 = 0; rq4 < 4; ++rq4) {
        f32x4 x = {oacc[db][4 * rq4] * inv, oacc[db][4 * rq4 + 1] * inv, oacc[db][4 * rq4 + 2] * inv,
                   oacc[db][4 * rq4 + 3] * inv};
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * rq4 + 4 * g) = to_bf16x4(x);
      }
  }
}

}  // namespace

template <int D, bool CAUSAL>
hipError_t launch_fwd(const FwdArgs& a) {
  const int nqb = (a.N + kFwdBR - 1) / kFwdBR;
  const int total = a.B * a.H * nqb;
  const float c2 = fabsf(a.scale) * kLog2e;
  const uint32_t q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL>), dim3(total), dim3(kFwdThreads), 0, a.stream,
                     static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                     static_cast<const bf16*>(a.v), static_cast<bf16*>(a.o), a.lse, a.N, a.H, nqb,
                     total, c2, q_sign);
  return hipGetLastError();
}

template hipError_t launch_fwd<64, false>(const FwdArgs&);
template hipError_t launch_fwd<64, true>(const FwdArgs&);
template hipError_t launch_fwd<128, false>(const FwdArgs&);
template hipError_t launch_fwd<128, true>(const FwdArgs&);

}  // namespace fa
