// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// Nq query rows against Nk key rows; with the causal mask key j is visible
// to query i iff j <= i + delta. f32_out selects a float32 output.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Nq, Nk, H;
  int delta;
  bool f32_out;
  float scale;
  hipStream_t stream;
  // Optional additive bias (bf16); element (b, h, i, j) at
  // bias[b * bias_sb + h * bias_sh + i * bias_srow + j]. Only with bf16 output.
  const void* bias = nullptr;
  long bias_sb = 0, bias_sh = 0;
  int bias_srow = 0;
};

struct MergeArgs {
  const float* o_parts;   // [C, B, N, H, d] float32
  const float* lse_parts; // [C, B, H, N] float32
  int C;
  void* o;                // [B, N, H, d] bfloat16
  float* lse;             // [B, H, N] float32
  int B, N, H;
  hipStream_t stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* lse2;    // [B, H, N] fp32 workspace, L * log2(e)
  float* dsum;    // [B, H, N] fp32 workspace, D = rowsum(dO * O)
  int B, N, H;
  float scale;
  hipStream_t stream;
  // Optional additive bias (as in FwdArgs) and its gradient dBias (bf16,
  // element (b, h, i, j) at dbias[((b * H + h) * N + i) * dbias_srow + j];
  // NULL: not computed).
  const void* bias = nullptr;
  long bias_sb = 0, bias_sh = 0;
  int bias_srow = 0;
  void* dbias = nullptr;
  int dbias_srow = 0;
};

template <int D, bool CAUSAL>
hipError_t launch_fwd(const FwdArgs& a);

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdArgs& a);

template <int D>
hipError_t launch_merge(const MergeArgs& a);

// FP8 (e4m3) forward, d = 64 or 128: q, k, v are e4m3 codes [B, N, H, d].
// Either one float32 descale per (batch, head) and tensor ([B, H]), or block
// scales (E8M0 bytes): q_scale, k_scale [B, N, H, d / 32] (one per 32
// consecutive d of a token), v_scale [B, ceil(N / 32), H, d] (one per 32
// consecutive tokens of a column).
struct Fp8Args {
  const void* q;
  const void* k;
  const void* v;
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  void* o;      // bf16 [B, N, H, d]
  float* lse;   // [B, H, N]
  int B, N, H;
  float scale;
  hipStream_t stream;
  const uint8_t* q_scale = nullptr;  // block scales (all three set: the microscaled form)
  const uint8_t* k_scale = nullptr;
  const uint8_t* v_scale = nullptr;
  int d = 128;                       // head dimension: 64 or 128
};

template <bool CAUSAL>
hipError_t launch_fwd_fp8(const Fp8Args& a);

// Decode-shaped attention: Nq query rows (the last Nq positions) against Nk
// keys, split into key ranges whose float32 results are merged.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* workspace;  // decode_workspace_bytes() bytes, 256-byte aligned
  int B, Nq, Nk, H;
  int delta;         // causal: key j visible to query i iff j <= i + delta
  float scale;
  hipStream_t stream;
};

template <int D, bool CAUSAL>
hipError_t launch_decode(const DecodeArgs& a);

// Keys per tile of the decode kernel; key ranges are multiples of it.
constexpr int kDecodeBC = 32;

// Key split of a decode call: enough (batch, head, range) workgroups to keep
// every CU streaming (about 2048 at d = 128, 4096 at d = 64, where a tile
// holds half the bytes), but ranges of at least 256 keys.
struct DecodeSplit {
  int nsplit, split_len;
};
inline DecodeSplit decode_split(long B, long Nq, long Nk, long H, long D) {
  const long kTargetBlocks = D == 64 ? 4096 : 2048, kMinKeys = 256;
  const long nqb = (Nq + 31) / 32;
  const long tiles = (Nk + kDecodeBC - 1) / kDecodeBC;
  const long units = B * H * nqb;
  long s = (kTargetBlocks + units - 1) / units;
  const long by_len = (Nk + kMinKeys - 1) / kMinKeys;
  if (s > by_len) s = by_len;
  if (s > tiles) s = tiles;
  if (s < 1) s = 1;
  const long len = (tiles + s - 1) / s * kDecodeBC;
  return {(int)((Nk + len - 1) / len), (int)len};
}
// Workspace of a split decode call: the float32 partial outputs
// [nsplit, B, Nq, H, d], then the partial logsumexps [nsplit, B, H, Nq],
// each padded to a multiple of 256 bytes.
inline long decode_part_elems(long elems) { return (elems + 63) / 64 * 64; }
inline size_t decode_workspace_bytes(long B, long Nq, long Nk, long H, long D) {
  const DecodeSplit sp = decode_split(B, Nq, Nk, H, D);
  if (sp.nsplit == 1) return 0;
  const long rows = B * Nq * H;
  return (size_t)(decode_part_elems(sp.nsplit * rows * D) + decode_part_elems(sp.nsplit * rows)) * 4;
}

// Workspace layout of the backward pass: L * log2(e), then D; each part is a
// float32 [B, H, N] array starting on a 256-byte boundary.
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline size_t bwd_row_bytes(long B, long N, long H) { return align256(size_t(B * H * N) * 4); }

}  // namespace fa
