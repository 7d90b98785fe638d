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
//
// Per wave and K/V tile (64 keys):
//   S^T = K Q^T     (MFMA; lane l owns query row l % 32, so a row's scores
//                    sit in two lanes: l and l ^ 32)
//   online softmax in the log2 domain: c2 = |scale| * log2(e) is folded into
//   one FMA per score before exp2; the row max and the rescale factor need a
//   single cross-half exchange; the running sum stays per lane and is only
//   combined in the epilogue; the division by the row sum is deferred to the
//   epilogue.
//   O^T += V^T P^T  (MFMA; P^T is taken straight from the S^T accumulator
//                    registers, V^T is read with LDS transpose loads)
// Causal masking: tiles entirely above the diagonal are never visited, and a
// wave skips tiles that are fully masked for its 32 rows; only tiles that
// straddle the diagonal (or the ragged end of the sequence) apply a mask.
// A negative softmax scale is handled by negating Q when it is loaded.

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kFwdBR = 128;     // query rows per workgroup
constexpr int kFwdBC = 64;      // keys per K/V tile
constexpr int kFwdThreads = 256;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads) void fwd_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int H, int nqb, int total_blocks,
    float c2, uint32_t q_sign) {
  constexpr int CH = D / 8;                        // 16-byte chunks per row
  constexpr int TILE = kFwdBC * D * 2;             // bytes of one K or V tile
  constexpr int LOADS = kFwdBC * CH / kFwdThreads; // 16-byte loads per thread per tile
  constexpr int KS = D / 16;                       // MFMA k-steps over d
  constexpr int DB = D / 32;                       // 32-wide output column blocks
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;

  const int logical = xcd_remap(blockIdx.x, total_blocks);
  const int head = logical / nqb;                  // b * H + h
  const int qblk = nqb - 1 - (logical - head * nqb);  // longest causal rows first
  const int b = head / H, h = head - b * H;
  const long tok = (long)H * D;                    // elements between tokens
  const long base = ((long)b * N * H + h) * D;
  const bf16* Qh = Q + base;
  const bf16* Kh = K + base;
  const bf16* Vh = V + base;

  const int qw0 = qblk * kFwdBR + wave * 32;       // first query row of this wave
  const int myq = qw0 + l32;

  // Q as the B operand of S^T = K Q^T: row myq, d = 16*ks + 8*g .. +7.
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (myq < N) x = *reinterpret_cast<const u32x4*>(Qh + myq * tok + 16 * ks + 8 * g);
    x ^= q_sign;
    qf[ks] = __builtin_bit_cast(bf16x8, x);
  }

  const int kv_len = CAUSAL ? min(N, (qblk + 1) * kFwdBR) : N;
  const int ntiles = (kv_len + kFwdBC - 1) / kFwdBC;

  u32x4 kreg[LOADS], vreg[LOADS];
  auto gload = [&](int tile) {
#pragma unroll
    for (int p = 0; p < LOADS; ++p) {
      const int cidx = tid + kFwdThreads * p;
      const int row = cidx / CH, c = cidx % CH;
      const int key = tile * kFwdBC + row;
      if (key < N) {
        kreg[p] = *reinterpret_cast<const u32x4*>(Kh + key * tok + c * 8);
        vreg[p] = *reinterpret_cast<const u32x4*>(Vh + key * tok + c * 8);
      } else {
        kreg[p] = u32x4{0u, 0u, 0u, 0u};
        vreg[p] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto swrite = [&](int buf) {
    char* kt = smem + buf * 2 * TILE;
    char* vt = kt + TILE;
#pragma unroll
    for (int p = 0; p < LOADS; ++p) {
      const int cidx = tid + kFwdThreads * p;
      const int row = cidx / CH, c = cidx % CH;
      lds_write16(kt, tile_off<D>(row, c), kreg[p]);
      lds_write16(vt, tile_off<D>(row, c), vreg[p]);
    }
  };

  gload(0);
  swrite(0);
  __syncthreads();

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running max of c2 * score (log2 domain)
  float l_run = 0.f;        // this lane's share of the running sum

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) gload(j + 1);
    const int key0 = j * kFwdBC;
    const bool active = !CAUSAL || key0 <= qw0 + 31;  // wave-uniform
    if (active) {
      const char* kt = smem + buf * 2 * TILE;
      const char* vt = kt + TILE;
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          s[kb] = mfma32(read_row8<D>(kt, kb * 32 + l32, 2 * ks + g), qf[ks], s[kb]);
      }
      const bool need_mask = (CAUSAL && key0 + kFwdBC - 1 > qw0) || (key0 + kFwdBC > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            const bool masked = (CAUSAL && key > myq) || key >= N;
            if (masked) s[kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = xhalf_max(mx);
      const float tile_m = (mx == -INFINITY) ? -INFINITY : mx * c2;
      const float m_new = fmaxf(m_run, tile_m);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;

      bf16x8 pf[4];
      float lsum = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        f32x8 p;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          const float sv = s[ks >> 1][8 * (ks & 1) + s8];
          float e = fast_exp2(__builtin_fmaf(sv, c2, -m_use));
          if (need_mask) e = (sv == -INFINITY) ? 0.f : e;
          p[s8] = e;
          lsum += e;
        }
        pf[ks] = to_bf16x8(p);
      }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

      const int G = lane >> 4;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 a = read_col8<D>(vt, 16 * ks + 4 * g, 16 * ks + 8 + 4 * g, 32 * db + 16 * (G & 1), lane);
          oacc[db] = mfma32(a, pf[ks], oacc[db]);
        }
    }
    if (j + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = xhalf_sum(l_run);
  const float inv = 1.f / l_tot;
  if (myq < N) {
    if (g == 0) LSE[(long)head * N + myq] = (m_run + log2f(l_tot)) * kLn2;
    bf16* orow = O + base + myq * tok;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4 x = {oacc[db][4 * rq] * inv, oacc[db][4 * rq + 1] * inv, oacc[db][4 * rq + 2] * inv,
                   oacc[db][4 * rq + 3] * inv};
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * rq + 4 * g) = to_bf16x4(x);
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
