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
};

template <int D, bool CAUSAL>
hipError_t launch_fwd(const FwdArgs& a);

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdArgs& a);

template <int D>
hipError_t launch_merge(const MergeArgs& a);

// Workspace layout of the backward pass: L * log2(e), then D; each part is a
// float32 [B, H, N] array starting on a 256-byte boundary.
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline size_t bwd_row_bytes(long B, long N, long H) { return align256(size_t(B * H * N) * 4); }

}  // namespace fa
