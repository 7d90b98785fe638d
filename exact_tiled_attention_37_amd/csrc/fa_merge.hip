// Merge of attention results computed over disjoint key chunks.
//
// The Ring Attention entry on the "High-Bandwidth Memory" keyword page
// computes attention block by block, each device's queries meeting one
// key/value block per pass; the IPLEX post on FlashAttention-2 work
// partitioning (section "Tiling preserves the attention calculation")
// requires blocks to combine into the globally normalised result. Each chunk
// c supplies its normalised output O_c and the natural-log logsumexp L_c of
// its scaled scores; the combination is
//     L = ln sum_c exp(L_c),   O = sum_c exp(L_c - L) O_c,
// computed with the largest L_c as the shift so no exponent is positive.
// Rows with L_c = -inf for every chunk saw no key: O = 0 and L = -inf.
//
// Memory-bound: per output row it reads C rows of d float32 plus C logsumexp
// values and writes d bfloat16 plus one float. Rows are laid out [B, N, H]
// in the outputs and in every chunk, so a wave reads whole contiguous rows;
// D / 4 lanes cover one row with 16-byte loads. A lane's loads of the C
// chunks are independent and are issued in batches (8 or 16); few rows with
// many chunks (decode-shaped calls, whose partial results were just
// written and come from memory rather than L2) would otherwise wait on one
// load latency per few chunks.
// Small row counts launch 64-thread workgroups, so that they still reach
// every CU.

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kMergeThreads = 256;       // threads per workgroup (64 for small launches)
constexpr int kMergeSmallThreads = 64;

// BATCH > 0 (small launches: few rows, often many chunks): the chunk loads
// are issued in explicit batches of BATCH, all in flight before any is used.
// BATCH = 0 (large, bandwidth-bound launches): plain loops unrolled by 8,
// which keep the register count low and the waves per SIMD high (batches
// measured slower there).
template <int D, int BATCH>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float* __restrict__ Op,
                                                               const float* __restrict__ Lp, int C,
                                                               bf16* __restrict__ O, float* __restrict__ L,
                                                               int N, int H, long rows) {
  constexpr int LPR = D / 4;                     // lanes per row
  const int rpb = (int)blockDim.x / LPR;         // rows per block
  const long r = (long)blockIdx.x * rpb + threadIdx.x / LPR;
  const int c4 = threadIdx.x % LPR;
  if (r >= rows) return;
  const int h = (int)(r % H);
  const long bn = r / H;
  const int n = (int)(bn % N);
  const long b = bn / N;
  const long lrow = (b * H + h) * N + n;         // index in a [B, H, N] array
  const long lstride = rows;                     // B * H * N = B * N * H
  const long ostride = rows * D;                 // elements per chunk of O

  // Batched form: all loads of a batch are issued before any is used (the
  // guards keep a short last batch, or a C below the batch size, in one round
  // trip too). Both forms add the chunks in order.
  float m = -INFINITY;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if constexpr (BATCH == 0) {
#pragma unroll 8
    for (int c = 0; c < C; ++c) m = fmaxf(m, Lp[c * lstride + lrow]);
    if (m != -INFINITY) {
      const float* op = Op + r * D + 4 * c4;
#pragma unroll 8
      for (int c = 0; c < C; ++c) {
        const float w = fast_exp2((Lp[c * lstride + lrow] - m) * kLog2e);  // exp2(-inf) = 0
        const f32x4 x = *reinterpret_cast<const f32x4*>(op + c * ostride);
        tot += w;
        acc += w * x;
      }
    }
  } else {
    for (int c0 = 0; c0 < C; c0 += BATCH) {
      float lb[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) lb[u] = c0 + u < C ? Lp[(c0 + u) * lstride + lrow] : -INFINITY;
#pragma unroll
      for (int u = 0; u < BATCH; ++u) m = fmaxf(m, lb[u]);
    }
    if (m != -INFINITY) {
      const float* op = Op + r * D + 4 * c4;
      for (int c0 = 0; c0 < C; c0 += BATCH) {
        float lb[BATCH];
        f32x4 xb[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
          if (c0 + u < C) {
            lb[u] = Lp[(c0 + u) * lstride + lrow];
            xb[u] = *reinterpret_cast<const f32x4*>(op + (c0 + u) * ostride);
          }
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
          if (c0 + u < C) {  // the chunks in order, as a plain loop over c would add them
            const float w = fast_exp2((lb[u] - m) * kLog2e);  // exp2(-inf) = 0
            tot += w;
            acc += w * xb[u];
          }
      }
    }
  }
  const bool seen = tot > 0.f;
  const float inv = seen ? 1.f / tot : 0.f;
  *reinterpret_cast<bf16x4*>(O + r * D + 4 * c4) = to_bf16x4(acc * inv);
  if (c4 == 0) L[lrow] = seen ? m + logf(tot) : -INFINITY;
}

}  // namespace

template <int D>
hipError_t launch_merge(const MergeArgs& a) {
  const long rows = (long)a.B * a.N * a.H;
  // Fewer than two full workgroups per CU: smaller workgroups spread the rows
  // over more CUs.
  const int threads =
      (rows + kMergeThreads / (D / 4) - 1) / (kMergeThreads / (D / 4)) < 2 * kNumXcd * kCusPerXcd ? kMergeSmallThreads
                                                                                                : kMergeThreads;
  const int rpb = threads / (D / 4);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (threads == kMergeSmallThreads)
    hipLaunchKernelGGL((merge_kernel<D, 16>), dim3(grid), dim3(threads), 0, a.stream, a.o_parts, a.lse_parts, a.C,
                       static_cast<bf16*>(a.o), a.lse, a.N, a.H, rows);
  else
    hipLaunchKernelGGL((merge_kernel<D, 0>), dim3(grid), dim3(threads), 0, a.stream, a.o_parts, a.lse_parts, a.C,
                       static_cast<bf16*>(a.o), a.lse, a.N, a.H, rows);
  return hipGetLastError();
}

template hipError_t launch_merge<64>(const MergeArgs&);
template hipError_t launch_merge<128>(const MergeArgs&);

}  // namespace fa
