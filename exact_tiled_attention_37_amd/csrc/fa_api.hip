// C ABI of the library: argument validation, device check and dispatch to the
// gfx950 kernels. Declarations and the full contract are in include/fa.h.

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "fa.h"
#include "fa_launch.hpp"

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int kMaxDevices = 64;
constexpr long long kMaxElems = (1LL << 31) - (1LL << 16);
constexpr int kMaxMergeChunks = 65536;

// 0 = not checked yet, 1 = gfx950, 2 = something else.
std::atomic<int> g_device_state[kMaxDevices];

fa_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_DEVICE;
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_HIP;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? FA_OK : FA_ERR_DEVICE;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

fa_status check_shape(int B, int N, int H, int d) {
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (B < 1 || N < 1 || H < 1) return FA_ERR_SHAPE;
  // Byte offsets within one sequence must stay below 2^32: buffer loads use
  // 32-bit offsets, and rows past the end are addressed at N * row bytes.
  const long long elems = (long long)B * N * H * d;
  if (elems > kMaxElems) return FA_ERR_SHAPE;
  return FA_OK;
}

template <typename F>
fa_status dispatch(int d, int causal, F&& f) {
  hipError_t e;
  if (d == 64)
    e = causal ? f(std::integral_constant<int, 64>{}, std::true_type{})
               : f(std::integral_constant<int, 64>{}, std::false_type{});
  else
    e = causal ? f(std::integral_constant<int, 128>{}, std::true_type{})
               : f(std::integral_constant<int, 128>{}, std::false_type{});
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

// Scratch of fa_decode_noalloc: the key-split partial results of a decode
// call, in place of a caller-supplied workspace. Every device the library
// runs on holds its own copy from module load until the process ends. Host
// code never uses the array's name as an address: the device address comes
// from hipGetSymbolAddress, taken once per device (with that device current)
// and kept in g_scratch.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// Validation shared by fa_decode and fa_decode_noalloc; on FA_OK *need holds
// the workspace bytes of the call.
fa_status check_decode(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                       int Nq, int Nk, int H, int d, float softmax_scale, size_t* need) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (B < 1 || Nq < 1 || Nk < 1 || H < 1) return FA_ERR_SHAPE;
  fa_status st = check_shape(B, Nq, H, d);
  if (st != FA_OK || (st = check_shape(B, Nk, H, d)) != FA_OK) return st;
  if (!std::isfinite(softmax_scale)) return FA_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  *need = fa::decode_workspace_bytes(B, Nq, Nk, H, d);
  return FA_OK;
}

fa_status launch_decode_checked(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Nq,
                                int Nk, int H, int d, int causal, float softmax_scale, void* workspace,
                                hipStream_t stream) {
  (void)hipGetLastError();
  // The queries are the last Nq positions: key j is visible to query i iff
  // j <= i + Nk - Nq (clamped as in fa_fwd_chunk; a single query sees all).
  int delta = 0;
  if (causal) {
    const long long dl = (long long)Nk - Nq;
    if (dl >= (long long)Nk - 1)
      causal = 0;
    else
      delta = (int)(dl < -(long long)Nq ? -(long long)Nq : dl);
  }
  const fa::DecodeArgs a{q, k, v, o, lse, static_cast<float*>(workspace), B, Nq, Nk, H, delta, softmax_scale, stream};
  return dispatch(d, causal, [&](auto D, auto C) { return fa::launch_decode<decltype(D)::value, decltype(C)::value>(a); });
}

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// This device's address of `scratch` (looked up on the first call per device).
fa_status scratch_address(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int N,
                 int H, int d, int causal, float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status st = check_shape(B, N, H, d);
  if (st != FA_OK) return st;
  if (!std::isfinite(softmax_scale)) return FA_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  st = check_device();
  if (st != FA_OK) return st;
  (void)hipGetLastError();  // do not report an earlier, unrelated error as ours
  const fa::FwdArgs a{q, k, v, o, lse, B, N, N, H, 0, false, softmax_scale, stream};
  return dispatch(d, causal, [&](auto D, auto C) { return fa::launch_fwd<decltype(D)::value, decltype(C)::value>(a); });
}

fa_status fa_fwd_chunk(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Nq,
                       int Nk, int H, int d, int causal, long long q_start, long long k_start,
                       float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (B < 1 || Nq < 1 || Nk < 0 || H < 1) return FA_ERR_SHAPE;
  fa_status st = check_shape(B, Nq, H, d);
  if (st != FA_OK) return st;
  if (Nk > 0 && (st = check_shape(B, Nk, H, d)) != FA_OK) return st;
  if (!std::isfinite(softmax_scale)) return FA_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  st = check_device();
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  // Causal: key j is visible to query i iff j <= i + delta. Clamping delta to
  // [-Nq, Nk - 1] keeps the same visible sets (below -Nq + 1 no row sees a
  // key; from Nk - 1 on every row sees every key, which is the unmasked case).
  int delta = 0;
  if (causal) {
    const long long dl = q_start - k_start;
    if (dl >= (long long)Nk - 1) {
      causal = 0;
    } else {
      delta = (int)(dl < -(long long)Nq ? -(long long)Nq : dl);
    }
  }
  const fa::FwdArgs a{q, k, v, o, lse, B, Nq, Nk, H, delta, true, softmax_scale, stream};
  return dispatch(d, causal, [&](auto D, auto C) { return fa::launch_fwd<decltype(D)::value, decltype(C)::value>(a); });
}

namespace {
// Bias layout checks shared by the biased entry points: row stride a multiple
// of 8 elements and at least N, batch/head strides multiples of 8 (0 =
// broadcast), 16-byte aligned base, and every (batch, head) slice addressable
// with 32-bit byte offsets.
fa_status check_bias(const void* bias, long long sb, long long sh, int srow, int N) {
  if (srow < N || srow % 8 != 0 || sb < 0 || sh < 0 || sb % 8 != 0 || sh % 8 != 0) return FA_ERR_SHAPE;
  if (((long long)N + 64) * srow * 2 >= (1LL << 32)) return FA_ERR_SHAPE;
  if (!aligned(bias, 16)) return FA_ERR_ALIGN;
  return FA_OK;
}
}  // namespace

fa_status fa_fwd_bias(const void* q, const void* k, const void* v, const void* bias, long long bias_stride_b,
                      long long bias_stride_h, int bias_stride_row, void* o, float* lse, int B, int N, int H,
                      int d, int causal, float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !bias || !o || !lse) return FA_ERR_NULL;
  fa_status st = check_shape(B, N, H, d);
  if (st != FA_OK) return st;
  if (!std::isfinite(softmax_scale)) return FA_ERR_SCALE;
  if ((st = check_bias(bias, bias_stride_b, bias_stride_h, bias_stride_row, N)) != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  st = check_device();
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  fa::FwdArgs a{q, k, v, o, lse, B, N, N, H, 0, false, softmax_scale, stream};
  a.bias = bias;
  a.bias_sb = (long)bias_stride_b;
  a.bias_sh = (long)bias_stride_h;
  a.bias_srow = bias_stride_row;
  return dispatch(d, causal, [&](auto D, auto C) { return fa::launch_fwd<decltype(D)::value, decltype(C)::value>(a); });
}

fa_status fa_bwd_bias(const void* q, const void* k, const void* v, const void* bias, long long bias_stride_b,
                      long long bias_stride_h, int bias_stride_row, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, void* dbias, int dbias_stride_row,
                      void* workspace, size_t workspace_bytes, int B, int N, int H, int d, int causal,
                      float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !bias || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  fa_status st = check_shape(B, N, H, d);
  if (st != FA_OK) return st;
  if (!std::isfinite(softmax_scale)) return FA_ERR_SCALE;
  if ((st = check_bias(bias, bias_stride_b, bias_stride_h, bias_stride_row, N)) != FA_OK) return st;
  if (dbias) {
    if (dbias_stride_row < N || dbias_stride_row % 8 != 0) return FA_ERR_SHAPE;
    if (!aligned(dbias, 16)) return FA_ERR_ALIGN;
  }
  if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, N, H, d)) return FA_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(workspace, 256))
    return FA_ERR_ALIGN;
  st = check_device();
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  char* ws = static_cast<char*>(workspace);
  fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv,
                reinterpret_cast<float*>(ws),
                reinterpret_cast<float*>(ws + fa::bwd_row_bytes(B, N, H)),
                B, N, H, softmax_scale, stream};
  a.bias = bias;
  a.bias_sb = (long)bias_stride_b;
  a.bias_sh = (long)bias_stride_h;
  a.bias_srow = bias_stride_row;
  a.dbias = dbias;
  a.dbias_srow = dbias_stride_row;
  return dispatch(d, causal, [&](auto D, auto C) { return fa::launch_bwd<decltype(D)::value, decltype(C)::value>(a); });
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale, const float* k_descale,
                     const float* v_descale, void* o, float* lse, int B, int N, int H, int d, int causal,
                     float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !q_descale || !k_descale || !v_descale || !o || !lse) return FA_ERR_NULL;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  fa_status st = check_shape(B, N, H, d);
  if (st != FA_OK) return st;
  if (!std::isfinite(softmax_scale)) return FA_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(q_descale, 4) || !aligned(k_descale, 4) || !aligned(v_descale, 4))
    return FA_ERR_ALIGN;
  st = check_device();
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  fa::Fp8Args a{q, k, v, q_descale, k_descale, v_descale, o, lse, B, N, H, softmax_scale, stream};
  a.d = d;
  const hipError_t e = causal ? fa::launch_fwd_fp8<true>(a) : fa::launch_fwd_fp8<false>(a);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_mxfp8(const void* q, const void* q_scale, const void* k, const void* k_scale, const void* v,
                       const void* v_scale, void* o, float* lse, int B, int N, int H, int d, int causal,
                       float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !q_scale || !k_scale || !v_scale || !o || !lse) return FA_ERR_NULL;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  fa_status st = check_shape(B, N, H, d);
  if (st != FA_OK) return st;
  if (!std::isfinite(softmax_scale)) return FA_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return FA_ERR_ALIGN;
  st = check_device();
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  fa::Fp8Args a{q, k, v, nullptr, nullptr, nullptr, o, lse, B, N, H, softmax_scale, stream};
  a.q_scale = static_cast<const uint8_t*>(q_scale);
  a.k_scale = static_cast<const uint8_t*>(k_scale);
  a.v_scale = static_cast<const uint8_t*>(v_scale);
  a.d = d;
  const hipError_t e = causal ? fa::launch_fwd_fp8<true>(a) : fa::launch_fwd_fp8<false>(a);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_decode_workspace_bytes(int B, int Nq, int Nk, int H, int d) {
  if (check_shape(B, Nq, H, d) != FA_OK || check_shape(B, Nk, H, d) != FA_OK) return 0;
  return fa::decode_workspace_bytes(B, Nq, Nk, H, d);
}

fa_status fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Nq, int Nk,
                    int H, int d, int causal, float softmax_scale, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  size_t need = 0;
  fa_status st = check_decode(q, k, v, o, lse, B, Nq, Nk, H, d, softmax_scale, &need);
  if (st != FA_OK) return st;
  if (need > 0 && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 256)) return FA_ERR_ALIGN;
  st = check_device();
  if (st != FA_OK) return st;
  return launch_decode_checked(q, k, v, o, lse, B, Nq, Nk, H, d, causal, softmax_scale, workspace, stream);
}

fa_status fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Nq,
                            int Nk, int H, int d, int causal, float softmax_scale, hipStream_t stream) {
  size_t need = 0;
  fa_status st = check_decode(q, k, v, o, lse, B, Nq, Nk, H, d, softmax_scale, &need);
  if (st != FA_OK) return st;
  if (need > kScratchBytes) return FA_ERR_SCRATCH;
  st = check_device();
  if (st != FA_OK) return st;
  void* ws = nullptr;
  if (need > 0 && (st = scratch_address(&ws)) != FA_OK) return st;
  return launch_decode_checked(q, k, v, o, lse, B, Nq, Nk, H, d, causal, softmax_scale, ws, stream);
}

fa_status fa_merge(const float* o_parts, const float* lse_parts, int C, void* o, float* lse, int B, int N,
                   int H, int d, hipStream_t stream) {
  if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_NULL;
  fa_status st = check_shape(B, N, H, d);
  if (st != FA_OK) return st;
  if (C < 1 || C > kMaxMergeChunks) return FA_ERR_SHAPE;
  if (!aligned(o_parts, 16) || !aligned(o, 16) || !aligned(lse_parts, 4) || !aligned(lse, 4)) return FA_ERR_ALIGN;
  st = check_device();
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  const fa::MergeArgs a{o_parts, lse_parts, C, o, lse, B, N, H, stream};
  const hipError_t e = d == 64 ? fa::launch_merge<64>(a) : fa::launch_merge<128>(a);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(int B, int N, int H, int d) {
  if (check_shape(B, N, H, d) != FA_OK) return 0;
  return 2 * fa::bwd_row_bytes(B, N, H);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int N, int H, int d, int causal,
                 float softmax_scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  fa_status st = check_shape(B, N, H, d);
  if (st != FA_OK) return st;
  if (!std::isfinite(softmax_scale)) return FA_ERR_SCALE;
  if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, N, H, d)) return FA_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 256))
    return FA_ERR_ALIGN;
  st = check_device();
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  char* ws = static_cast<char*>(workspace);
  fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv,
                reinterpret_cast<float*>(ws),
                reinterpret_cast<float*>(ws + fa::bwd_row_bytes(B, N, H)),
                B, N, H, softmax_scale, stream};
  return dispatch(d, causal, [&](auto D, auto C) { return fa::launch_bwd<decltype(D)::value, decltype(C)::value>(a); });
}

const char* fa_status_string(fa_status status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape: B, N, H must be >= 1 and B*N*H*d <= 2^31 - 2^16";
    case FA_ERR_HEADDIM: return "unsupported head dimension: d must be 64 or 128";
    case FA_ERR_ALIGN: return "misaligned pointer: tensors need 16 bytes, lse 4, workspace 256";
    case FA_ERR_SCALE: return "softmax_scale is not finite";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than fa_bwd_workspace_bytes()";
    case FA_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case FA_ERR_DEVICE: return "the current device is not a gfx950 (MI355X) GPU";
    case FA_ERR_SCRATCH: return "the call needs more scratch than fa_decode_noalloc holds (32 MiB): use fa_decode";
  }
  return "unknown status";
}

int fa_version(void) { return kVersion; }

}  // extern "C"
