// Device-side building blocks shared by the forward and backward kernels
// (gfx950 / CDNA4 only).
//
// Register layouts used throughout (verified on the device for
// v_mfma_f32_32x32x16_bf16, lane l, g = l / 32):
//   A operand (32 x 16, M x K): lane l holds row m = l % 32, k = 8g .. 8g+7
//   B operand (16 x 32, K x N): lane l holds column n = l % 32, k = 8g .. 8g+7
//   C/D (32 x 32):              lane l holds column n = l % 32 and rows
//                               m = 8*(r/4) + 4g + (r%4) for r = 0..15
// Only the pairing of A's and B's k slots matters for the product, so an
// operand may present its k values in any order as long as the other operand
// uses the same order.
//
// LDS tiles (see Tile below) store a row-major R x D bfloat16 block as
// 1 KiB blocks of 16 rows x 4 chunks (a chunk is 16 bytes: 8 elements of a
// row), with the chunk order inside each 64-byte row slice XOR-swizzled by
// row / 4. Then:
//   * a whole-wave LDS-direct load of 1 KiB fills one block from 16 rows x
//     64 contiguous bytes of memory;
//   * row reads (16 lanes read the same chunk of 16 consecutive rows) and
//     transpose reads (ds_read_b64_tr_b16: a 16-lane group reads two
//     adjacent chunks of 4 consecutive rows, the next group the next two
//     chunks of the same rows) hit 16 distinct 16-byte bank slots, i.e. no
//     bank conflicts;
//   * every LDS address is one of two per-lane bases plus a compile-time
//     offset, so the reads need no address arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, one L2 each

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x32_bf16, lane l, G = l / 16:
//   A operand (16 x 32, M x K): lane l holds row m = l % 16, k = 8G .. 8G+7
//   B operand (32 x 16, K x N): lane l holds column n = l % 16, k = 8G .. 8G+7
//   C/D (16 x 16):              lane l holds column n = l % 16, rows 4G .. 4G+3
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Generic pointers into __shared__ arrays are converted to LDS (address
// space 3) pointers so that ds_read / ds_write instructions are emitted.
__device__ __forceinline__ u32x4 lds_read16(const char* base, int off) {
  return *(const FA_LDS u32x4*)((const FA_LDS char*)base + off);
}
__device__ __forceinline__ void lds_write16(char* base, int off, u32x4 v) {
  *(FA_LDS u32x4*)((FA_LDS char*)base + off) = v;
}
__device__ __forceinline__ void lds_write8(char* base, int off, u32x2 v) {
  *(FA_LDS u32x2*)((FA_LDS char*)base + off) = v;
}

// ds_read_b64_tr_b16: within each 16-lane group, lane t supplies the address
// of 4 consecutive 16-bit elements ("chunk t"); lane j receives element
// j%4 of chunks j/4, j/4+4, j/4+8, j/4+12 (measured on the device).
__device__ __forceinline__ i16x4 lds_read_tr(const char* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)((FA_LDS char*)base + off));
}

// LDS tile of R rows (R = 32, 64 or 128) by D bfloat16 columns, laid out as
// described at the top of this file: block (row / 16, chunk / 4) at
// ((row / 16) * (D / 32) + chunk / 4) * 1024 bytes; inside a block, row r
// (0..15) and chunk c (0..3) sit in 16-byte slot 4 r + (c ^ s(r)) with
// s(r) = r / 4. SWAP: s(r) = (r / 2) % 4, for waves whose four 16-lane
// groups read four different chunks of the same 16 rows (row reads) or
// four consecutive rows each, 4 rows apart, at the same columns (transpose
// reads). Measured with the LDS bank-conflict counter on a probe of exactly
// those reads: with s(r) = r / 4 every ds_read_b128 of the row pattern
// costs 4 conflict cycles and every ds_read_b64_tr_b16 of the transpose
// pattern 2; with (r / 2) % 4 neither conflicts. (The 32-row waves' reads,
// 32 consecutive rows per chunk, are conflict-free with r / 4.)
template <int R, int D, bool SWAP = false>
struct Tile {
  static_assert(R == 32 || R == 64 || R == 128, "tile rows");
  static_assert(D == 64 || D == 128, "head dimension");
  static constexpr int CH = D / 8;      // chunks per row
  static constexpr int NCB = CH / 4;    // 4-chunk blocks per row
  static constexpr int BYTES = R * D * 2;
  static constexpr int LOADS = BYTES / 1024;  // whole-wave 1 KiB loads per tile

  // the chunk swizzle of row rl (0..15) of a block
  __device__ static constexpr int swz(int rl) { return SWAP ? (rl >> 1) & 3 : rl >> 2; }
  __device__ static constexpr int addr(int row, int c) {
    const int rl = row & 15;
    return (((row >> 4) * NCB + (c >> 2)) << 10) + ((rl << 2) + ((c & 3) ^ swz(rl))) * 16;
  }
  // Whole-wave load u fills block u (bytes [1024 u, 1024 u + 1024)); lane i
  // writes slot i, which holds chunk dma_chunk of row dma_row.
  __device__ static constexpr int dma_dst(int u) { return u << 10; }
  __device__ static constexpr int dma_row(int u, int lane) { return (u / NCB) * 16 + (lane >> 2); }
  __device__ static constexpr int dma_chunk(int u, int lane) {
    return (u % NCB) * 4 + ((lane & 3) ^ swz(lane >> 2));
  }

  // Byte offset in memory (rows row_bytes apart) of what lane `lane` loads
  // for whole-wave load u, split into a part that depends only on the lane
  // and a part that depends only on u (wave-uniform).
  __device__ static uint32_t dma_lane_off(int lane, uint32_t row_bytes) {
    return (uint32_t)(lane >> 2) * row_bytes + 16u * (uint32_t)((lane & 3) ^ swz(lane >> 2));
  }
  __device__ static uint32_t dma_load_off(int u, uint32_t row_bytes) {
    return (uint32_t)(u / NCB) * 16u * row_bytes + 64u * (uint32_t)(u % NCB);
  }

  // Row read: chunk c (elements 8c..8c+7) of row `row`.
  __device__ static bf16x8 row8(const char* t, int row, int c) {
    return __builtin_bit_cast(bf16x8, lds_read16(t, addr(row, c)));
  }
  // Column read through two transpose loads: for this lane's column
  // col0 + (lane % 16) the 8 elements of rows rowA..rowA+3, rowB..rowB+3
  // (rowA/rowB given for the lane's 16-lane group and multiples of 4; col0 a
  // multiple of 16).
  __device__ static bf16x8 col8(const char* t, int rowA, int rowB, int col0, int lane) {
    const int j = lane & 15;
    const int col = col0 + 4 * (j & 3);
    const int c = col >> 3, half = (col >> 2) & 1;
    i16x4 lo = lds_read_tr(t, addr(rowA + (j >> 2), c) + 8 * half);
    i16x4 hi = lds_read_tr(t, addr(rowB + (j >> 2), c) + 8 * half);
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// Maxima that propagate NaN (IEEE maximum; v_maximum3_f32 on gfx950). fmaxf
// would make the compiler quiet possible signalling NaNs in every operand
// first (one extra v_max_f32 per MFMA result).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// Combine a value with the same value of lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float xhalf_max(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Combine a value over the four lanes l, l ^ 16, l ^ 32, l ^ 48
// (v_permlane16_swap, then v_permlane32_swap).
__device__ __forceinline__ float xquad_max(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return xhalf_max(vmax(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float xquad_sum(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return xhalf_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the values of an MFMA accumulator as two independent
// chains (short dependency depth): 8 three-input maxima for 16 values and init.
__device__ __forceinline__ float max16(const f32x16& v, float init) {
  float a = vmax3(v[0], v[1], v[2]);
  float b = vmax3(v[8], v[9], v[10]);
  a = vmax3(a, v[3], v[4]);
  b = vmax3(b, v[11], v[12]);
  a = vmax3(a, v[5], v[6]);
  b = vmax3(b, v[13], v[14]);
  return vmax3(vmax3(a, v[7], v[15]), b, init);
}
__device__ __forceinline__ float sum8(const f32x8& v) {
  return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

// Byte offset of row `row` (chunk offset col) inside a buffer resource made
// over rows [0, n): rows at or past n are clamped to n, whose offset is
// already past the resource's end, so they read as zeros. n * row_bytes must
// stay below 2^32 (guaranteed by the element limit the library enforces).
__device__ __forceinline__ uint32_t row_off(int row, int n, uint32_t row_bytes, uint32_t col) {
  return (uint32_t)min(row, n) * row_bytes + col;
}

// Buffer resource over `nbytes` bytes starting at `base`. Loads whose byte
// offset falls outside [0, nbytes) return zeros (the hardware range check),
// which is how rows past the end of a sequence are read.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// voff: per-lane byte offset; soff: wave-uniform byte offset (a scalar
// register operand of the load, so uniform address terms cost no VALU).
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint32_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}

// bfloat16 element e (0..3) of four packed in two dwords, as float32 (exact).
__device__ __forceinline__ float bf16_elem(const u32x2& w, int e) {
  const uint32_t x = w[e >> 1];
  return __builtin_bit_cast(float, (e & 1) ? (x & 0xFFFF0000u) : (x << 16));
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }

// The four descriptor words of the same resource, held in scalar registers,
// for the loads below that are written as inline assembly.
__device__ __forceinline__ u32x4 make_raw_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(nbytes);
  r[3] = 0x00020000u;
  return r;
}

// Loads straight from memory into LDS (no registers): lane i of the wave
// writes LDS bytes [lds + W i, lds + W i + W) for W = 16 (dma16) or 4
// (dma4); `lds` must be the same for the whole wave (it goes to M0).
//
// They are written as inline assembly on purpose. For the intrinsic form the
// compiler tracks only a few LDS-DMA writes individually and otherwise
// assumes that any pending one may alias a later LDS read, so it waits for
// the prefetch of the next tile before reading the current one, which
// serialises the pipeline. Here the loads are ordered only by the explicit
// vmcnt waits placed before each barrier (wait_vmem / wait_vmem_leave); the
// compiler's own vmcnt waits for register loads stay correct, because extra
// loads only make a "at most n outstanding" wait stricter.
__device__ __forceinline__ uint32_t lds_base(const void* lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const FA_LDS void*)lds);
}
__device__ __forceinline__ void dma16(const u32x4& r, const void* lds, uint32_t off) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds_base(lds)) : "memory");
}
__device__ __forceinline__ void dma4(const u32x4& r, const void* lds, uint32_t off) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds_base(lds)) : "memory");
}

// The same resource advanced by `off` bytes (wave-uniform): the base moves
// up and the record count shrinks by `off`, so a per-lane offset relative to
// the new base is range-checked against the same end. The values stay in
// scalar registers, which keeps per-tile address arithmetic off the VALU.
__device__ __forceinline__ u32x4 rsrc_advance(const u32x4& r, uint32_t off) {
  const uint64_t base = (((uint64_t)r[1] << 32) | r[0]) + off;
  u32x4 o;
  o[0] = __builtin_amdgcn_readfirstlane((uint32_t)base);
  o[1] = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  o[2] = __builtin_amdgcn_readfirstlane(r[2] - off);
  o[3] = r[3];
  return o;
}
// dma16 with the LDS destination given as an LDS byte address (uniform).
__device__ __forceinline__ void dma16_at(const u32x4& r, uint32_t lds_addr, uint32_t off) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

__device__ __forceinline__ void dma4_at(const u32x4& r, uint32_t lds_addr, uint32_t off) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(r),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// s_waitcnt vmcnt(0): all of this wave's vector memory loads (including the
// ones that write LDS directly) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): all but this wave's N most recent vector memory loads
// have completed (loads complete in issue order for this counter).
template <int N>
__device__ __forceinline__ void wait_vmem_leave() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Blocks are dispatched round-robin over the XCDs (block i goes to XCD i % 8)
// and, inside an XCD, start in index order.
//
// xcd_remap: each XCD receives one contiguous range of logical blocks, so
// consecutive logical blocks (the blocks of one head) share an L2. The map
// is a bijection of [0, total) for any total, so correctness never depends
// on the dispatch order.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int per = total / kNumXcd, rem = total % kNumXcd;
  const int x = bid % kNumXcd, idx = bid / kNumXcd;
  return (x < rem) ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
}

// Block order of a launch over `heads` (batch, head) pairs with per_head
// blocks each; rank 0 is the block with the most work. The logical order
// (xcd_remap: one contiguous range per XCD) takes the heads in groups of G;
// inside a group the blocks go rank-major (heaviest rank of every head of
// the group first). Causal blocks of one head differ in work: with G chosen
// so that a group holds at least `rounds` times as many blocks as an XCD
// runs at once (`slots`), every XCD runs longest-first within the group (the
// head-by-head order left a head's heavy blocks behind the previous head's
// light ones), while only about G heads share the XCD's L2 at a time. The
// forward and backward kernels take two rounds per group (one left the next
// group's heavy blocks behind the current group's light ones), decode one.
// Non-causal blocks do equal work: G = 1, the blocks of a head run together
// and read their K and V through one L2.
struct HeadRank {
  int head, rank;
};
constexpr int kCusPerXcd = 32;  // MI355X: 256 CUs in 8 XCDs
template <bool CAUSAL>
__device__ __forceinline__ HeadRank block_order(int bid, int heads, int per_head, int slots, int rounds) {
  const int l = xcd_remap(bid, heads * per_head);
  int G = CAUSAL ? min(heads, max(1, (rounds * slots + per_head - 1) / per_head)) : 1;
  // A group must not straddle two XCDs' ranges of heads: the XCD holding its
  // first part would get only its heaviest blocks, the next one only its
  // lightest. With whole heads per XCD, G becomes the heads per XCD when it
  // is at least that many; a G that does not divide them becomes the next
  // power of two if that divides them (or reaches them). Other counts keep
  // G (one candidate only: this runs in every thread at the start).
  if (CAUSAL && heads % kNumXcd == 0) {
    const int hx = heads / kNumXcd;
    if (G >= hx) {
      G = hx;
    } else if (hx % G != 0) {  // then G > 1
      const int p2 = 1 << (32 - __builtin_clz((unsigned)(G - 1)));
      if (p2 >= hx)
        G = hx;
      else if (hx % p2 == 0)
        G = p2;
    }
  }
  const int gsize = G * per_head;
  const int g = l / gsize;
  const int within = l - g * gsize;
  const int gh = min(G, heads - g * G);  // heads in this group (the last may be smaller)
  const int r = within / gh;
  return {g * G + (within - r * gh), r};
}

}  // namespace fa
