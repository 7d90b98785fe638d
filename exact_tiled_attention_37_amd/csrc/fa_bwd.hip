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
// No N x N matrix is stored: every tile of P and dS lives in registers (and
// one 128 x 32 tile of dS in LDS) only.
//
// Three kernels, all on the caller's stream:
//   1. pre-pass: D = rowsum(dO * O) per query row; zeroes the fp32 dQ
//      accumulator (a kernel rather than a memset, so the call can be
//      captured in a graph).
//   2. main: one workgroup per (block of 128 keys, head, batch); each of the
//      4 wavefronts owns 32 keys, keeps its K and V rows in registers and its
//      dK, dV accumulators in registers, and streams 32-row blocks of Q and
//      dO through double-buffered LDS. Per step and wave:
//        S = Q K^T, dP = dO V^T           (lane l owns key l % 32)
//        P, dS elementwise                (L and D per row from LDS)
//        dV^T += dO^T P, dK^T += Q^T dS   (dO^T, Q^T by LDS transpose reads;
//                                          P, dS straight from registers)
//      dS is then written transposed to LDS, and the workgroup computes its
//      contribution to dQ of the 32 rows (dS K over its 128 keys), which is
//      added to the fp32 accumulator with hardware float atomics.
//   3. finalize: dQ = bf16(scale * accumulator).
// Causal: a key block only visits query blocks at or below the diagonal,
// waves skip steps that are fully masked for their keys, and only steps on
// the diagonal apply the mask. A negative scale negates Q on load, as in the
// forward pass.

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kBwdBKV = 128;  // keys per workgroup (4 waves x 32)
constexpr int kBwdBQ = 32;    // query rows per step
constexpr int kBwdThreads = 256;

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O); zero the dQ accumulator. Eight lanes per token row.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ O,
                                                       const bf16* __restrict__ dO,
                                                       float* __restrict__ dsum,
                                                       float* __restrict__ dq_acc, int N, int H,
                                                       long rows) {
  constexpr int PER = D / 8;  // elements per lane
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long r = t >> 3;      // token row (b, n, h), memory order
  const int sub = threadIdx.x & 7;
  if (r >= rows) return;      // all 8 lanes of a row leave together
  const long off = r * D + sub * PER;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < PER / 8; ++c) {
    const bf16x8 o8 = *reinterpret_cast<const bf16x8*>(O + off + 8 * c);
    const bf16x8 d8 = *reinterpret_cast<const bf16x8*>(dO + off + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)o8[e], (float)d8[e], acc);
  }
  acc += __shfl_xor(acc, 1, 8);
  acc += __shfl_xor(acc, 2, 8);
  acc += __shfl_xor(acc, 4, 8);
  if (sub == 0) {
    const long bn = r / H;
    const int h = (int)(r - bn * H);
    const long b = bn / N;
    const long n = bn - b * N;
    dsum[(b * H + h) * N + n] = acc;
  }
#pragma unroll
  for (int c = 0; c < PER / 4; ++c)
    *reinterpret_cast<f32x4*>(dq_acc + off + 4 * c) = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------------------
// 2. Main kernel.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void bwd_main_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dsum,
    float* __restrict__ dQacc, bf16* __restrict__ dK, bf16* __restrict__ dV, int N, int H,
    int nkb, int total_blocks, float c2, uint32_t q_sign, float dk_scale) {
  constexpr int CH = D / 8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int QT = kBwdBQ * D * 2;          // bytes of one Q or dO tile
  constexpr int KT = kBwdBKV * D * 2;         // bytes of the K tile
  constexpr int ST = kBwdBKV * kBwdBQ * 2;    // bytes of the dS^T tile
  constexpr int QLOADS = kBwdBQ * CH / kBwdThreads;
  constexpr int KLOADS = kBwdBKV * CH / kBwdThreads;
  __shared__ __attribute__((aligned(16))) char smem[4 * QT + KT + ST];
  __shared__ __attribute__((aligned(16))) float srow[2][2][kBwdBQ];  // [buf][L*log2e, D][row]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, G = lane >> 4;

  const int logical = xcd_remap(blockIdx.x, total_blocks);
  const int head = logical / nkb;
  const int kblk = logical - head * nkb;  // block 0 has the most causal work: it goes first
  const int b = head / H, h = head - b * H;
  const long tok = (long)H * D;
  const long base = ((long)b * N * H + h) * D;
  const bf16* Qh = Q + base;
  const bf16* Kh = K + base;
  const bf16* Vh = V + base;
  const bf16* dOh = dO + base;
  const float* Lh = LSE + (long)head * N;
  const float* Dh = Dsum + (long)head * N;

  const int kb0 = kblk * kBwdBKV;
  const int kw0 = kb0 + 32 * wave;
  const int mykey = kw0 + l32;

  char* const ktile = smem + 4 * QT;
  char* const stile = ktile + KT;

  // This wave's K and V rows as B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (mykey < N) {
      x = *reinterpret_cast<const u32x4*>(Kh + mykey * tok + 16 * ks + 8 * g);
      y = *reinterpret_cast<const u32x4*>(Vh + mykey * tok + 16 * ks + 8 * g);
    }
    kf[ks] = __builtin_bit_cast(bf16x8, x);
    vf[ks] = __builtin_bit_cast(bf16x8, y);
  }
  // The whole key block in LDS, for the dQ product.
#pragma unroll
  for (int p = 0; p < KLOADS; ++p) {
    const int cidx = tid + kBwdThreads * p;
    const int row = cidx / CH, c = cidx % CH;
    const int key = kb0 + row;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (key < N) x = *reinterpret_cast<const u32x4*>(Kh + key * tok + c * 8);
    lds_write16(ktile, tile_off<D>(row, c), x);
  }

  const int nqs = (N + kBwdBQ - 1) / kBwdBQ;
  const int qs_begin = CAUSAL ? kb0 / kBwdBQ : 0;

  u32x4 qreg[QLOADS], doreg[QLOADS];
  float rowv = 0.f;
  auto gload = [&](int step) {
#pragma unroll
    for (int p = 0; p < QLOADS; ++p) {
      const int cidx = tid + kBwdThreads * p;
      const int row = cidx / CH, c = cidx % CH;
      const int q = step * kBwdBQ + row;
      if (q < N) {
        qreg[p] = *reinterpret_cast<const u32x4*>(Qh + q * tok + c * 8) ^ q_sign;
        doreg[p] = *reinterpret_cast<const u32x4*>(dOh + q * tok + c * 8);
      } else {
        qreg[p] = u32x4{0u, 0u, 0u, 0u};
        doreg[p] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < 2 * kBwdBQ) {
      const int q = step * kBwdBQ + (tid & (kBwdBQ - 1));
      if (tid < kBwdBQ)
        rowv = (q < N) ? Lh[q] * kLog2e : INFINITY;  // P = 0 for rows past the end
      else
        rowv = (q < N) ? Dh[q] : 0.f;
    }
  };
  auto swrite = [&](int buf) {
    char* qt = smem + buf * 2 * QT;
    char* dot = qt + QT;
#pragma unroll
    for (int p = 0; p < QLOADS; ++p) {
      const int cidx = tid + kBwdThreads * p;
      const int row = cidx / CH, c = cidx % CH;
      lds_write16(qt, tile_off<D>(row, c), qreg[p]);
      lds_write16(dot, tile_off<D>(row, c), doreg[p]);
    }
    if (tid < 2 * kBwdBQ) srow[buf][tid / kBwdBQ][tid & (kBwdBQ - 1)] = rowv;
  };

  f32x16 dvacc[DB], dkacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dvacc[i] = f32x16{};
    dkacc[i] = f32x16{};
  }

  if (qs_begin < nqs) {
    gload(qs_begin);
    swrite(0);
  }
  __syncthreads();

  for (int step = qs_begin; step < nqs; ++step) {
    const int buf = (step - qs_begin) & 1;
    if (step + 1 < nqs) gload(step + 1);
    const int q0 = step * kBwdBQ;
    const char* qt = smem + buf * 2 * QT;
    const char* dot = qt + QT;
    const float* l2 = srow[buf][0];
    const float* dd = srow[buf][1];

    const bool active = !CAUSAL || kw0 <= q0 + kBwdBQ - 1;  // wave-uniform
    if (active) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(read_row8<D>(qt, l32, 2 * ks + g), kf[ks], s);
        dp = mfma32(read_row8<D>(dot, l32, 2 * ks + g), vf[ks], dp);
      }
      const bool need_mask = (CAUSAL && kw0 + 31 > q0) || (kw0 + 32 > N);
      f32x16 pv, dsv;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 8 * (r >> 2) + 4 * g + (r & 3);
        float p = fast_exp2(__builtin_fmaf(s[r], c2, -l2[qi]));
        if (need_mask && ((CAUSAL && mykey > q0 + qi) || mykey >= N)) p = 0.f;
        pv[r] = p;
        dsv[r] = p * (dp[r] - dd[qi]);
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f32x8 a, c;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          a[e] = pv[8 * hh + e];
          c[e] = dsv[8 * hh + e];
        }
        pb[hh] = to_bf16x8(a);
        dsb[hh] = to_bf16x8(c);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col0 = 32 * db + 16 * (G & 1);
          const bf16x8 a_do = read_col8<D>(dot, 16 * hh + 4 * g, 16 * hh + 8 + 4 * g, col0, lane);
          dvacc[db] = mfma32(a_do, pb[hh], dvacc[db]);
          const bf16x8 a_q = read_col8<D>(qt, 16 * hh + 4 * g, 16 * hh + 8 + 4 * g, col0, lane);
          dkacc[db] = mfma32(a_q, dsb[hh], dkacc[db]);
        }
      // dS^T rows of this wave's keys: row = key, columns = the 32 query rows.
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const bf16x4 v4 = to_bf16x4(f32x4{dsv[4 * rq], dsv[4 * rq + 1], dsv[4 * rq + 2], dsv[4 * rq + 3]});
        lds_write8(stile, tile_off<32>(32 * wave + l32, rq) + 8 * g, __builtin_bit_cast(u32x2, v4));
      }
    } else {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        lds_write8(stile, tile_off<32>(32 * wave + l32, rq) + 8 * g, u32x2{0u, 0u});
    }
    __syncthreads();

    // dQ rows q0..q0+31 += dS K over this block's keys (fp32 atomics).
    {
      constexpr int STEPS = (D == 128) ? 8 : 4;
      const int db = (D == 128) ? wave : (wave & 1);
      const int kbase = (D == 128) ? 0 : 64 * (wave >> 1);
      f32x16 dq = f32x16{};
#pragma unroll
      for (int t = 0; t < STEPS; ++t) {
        const int kr = kbase + 16 * t;
        const bf16x8 a = read_col8<32>(stile, kr + 4 * g, kr + 8 + 4 * g, 16 * (G & 1), lane);
        const bf16x8 bk = read_col8<D>(ktile, kr + 4 * g, kr + 8 + 4 * g, 32 * db + 16 * (G & 1), lane);
        dq = mfma32(a, bk, dq);
      }
      float* dqh = dQacc + base + 32 * db + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (q < N) unsafeAtomicAdd(dqh + q * tok, dq[r]);
      }
    }
    if (step + 1 < nqs) swrite(buf ^ 1);
    __syncthreads();
  }

  if (mykey < N) {
    bf16* dkrow = dK + base + mykey * tok;
    bf16* dvrow = dV + base + mykey * tok;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * db + 8 * rq + 4 * g;
        const f32x4 k4 = {dkacc[db][4 * rq] * dk_scale, dkacc[db][4 * rq + 1] * dk_scale,
                          dkacc[db][4 * rq + 2] * dk_scale, dkacc[db][4 * rq + 3] * dk_scale};
        const f32x4 v4 = {dvacc[db][4 * rq], dvacc[db][4 * rq + 1], dvacc[db][4 * rq + 2],
                          dvacc[db][4 * rq + 3]};
        *reinterpret_cast<bf16x4*>(dkrow + d0) = to_bf16x4(k4);
        *reinterpret_cast<bf16x4*>(dvrow + d0) = to_bf16x4(v4);
      }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ = bf16(scale * accumulator), 8 elements per thread.
__global__ __launch_bounds__(256) void bwd_finalize_kernel(const float* __restrict__ acc,
                                                            bf16* __restrict__ dq, float scale,
                                                            long n8) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(acc + 8 * i);
  const f32x4 c = *reinterpret_cast<const f32x4*>(acc + 8 * i + 4);
  const f32x8 x = {a[0] * scale, a[1] * scale, a[2] * scale, a[3] * scale,
                   c[0] * scale, c[1] * scale, c[2] * scale, c[3] * scale};
  *reinterpret_cast<bf16x8*>(dq + 8 * i) = to_bf16x8(x);
}

}  // namespace

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdArgs& a) {
  const long rows = (long)a.B * a.N * a.H;
  {
    const long threads = rows * 8;
    const unsigned grid = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3(grid), dim3(256), 0, a.stream,
                       static_cast<const bf16*>(a.o), static_cast<const bf16*>(a.dout), a.dsum,
                       a.dq_acc, a.N, a.H, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nkb = (a.N + kBwdBKV - 1) / kBwdBKV;
    const int total = a.B * a.H * nkb;
    const float c2 = fabsf(a.scale) * kLog2e;
    const uint32_t q_sign = a.scale < 0.f ? 0x80008000u : 0u;
    hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), dim3(total), dim3(kBwdThreads), 0, a.stream,
                       static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                       static_cast<const bf16*>(a.v), static_cast<const bf16*>(a.dout), a.lse,
                       a.dsum, a.dq_acc, static_cast<bf16*>(a.dk), static_cast<bf16*>(a.dv), a.N,
                       a.H, nkb, total, c2, q_sign, fabsf(a.scale));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const long n8 = rows * D / 8;
    const unsigned grid = (unsigned)((n8 + 255) / 256);
    hipLaunchKernelGGL(bwd_finalize_kernel, dim3(grid), dim3(256), 0, a.stream, a.dq_acc,
                       static_cast<bf16*>(a.dq), a.scale, n8);
    return hipGetLastError();
  }
}

template hipError_t launch_bwd<64, false>(const BwdArgs&);
template hipError_t launch_bwd<64, true>(const BwdArgs&);
template hipError_t launch_bwd<128, false>(const BwdArgs&);
template hipError_t launch_bwd<128, true>(const BwdArgs&);

}  // namespace fa
