/*
 * fa.h -- C ABI of the MI355X (gfx950) exact tiled attention library.
 *
 * The library computes exact scaled-dot-product attention the way the
 * FlashAttention-2 abstract (on the "High-Bandwidth Memory" keyword page)
 * and the IPLEX blog post on FlashAttention-2 GPU work partitioning describe
 * it: Q/K/V tiles are staged on chip, an online softmax keeps running row
 * statistics and rescales partial outputs (post section "Tiling preserves the
 * attention calculation"), no N x N score or probability matrix is written to
 * device memory, work is spread over batch x heads x query blocks and the
 * query rows of a block are split across wavefronts that share the K/V tiles
 * (section "Three changes improve GPU utilisation").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   - All tensor arguments are DEVICE pointers on the current HIP device.
 *   - q, k, v, o, dout, dq, dk, dv: bfloat16, contiguous, layout [B, N, H, d]
 *     (token-major: element (b, n, h, j) is at ((b*N + n)*H + h)*d + j).
 *     They must be 16-byte aligned.
 *   - lse: float32, contiguous, layout [B, H, N]; natural-log logsumexp of the
 *     scaled scores of each query row, L_i = ln sum_j exp(scale * q_i . k_j)
 *     over the visible keys j. 4-byte aligned.
 *   - Causal: key j is visible to query i iff j <= i (equal query and key
 *     lengths). Non-causal: every key is visible.
 *   - softmax_scale: any finite float (1/sqrt(d) is the usual choice).
 *   - Supported head dimensions: d = 64 and d = 128. Any N >= 1, B >= 1,
 *     H >= 1 with B*N*H*d <= 2^31 - 2^16.
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     without synchronising. Device faults surface at the caller's next
 *     synchronisation. Validation happens before anything is enqueued; a
 *     non-FA_OK status means nothing was launched.
 *   - The library allocates no device memory and keeps no per-call state;
 *     the caller owns every buffer. Calls on different streams may run
 *     concurrently as long as their output buffers do not overlap.
 *   - Outputs must not alias inputs.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifndef FA_API
#define FA_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer is NULL                         */
    FA_ERR_SHAPE = 2,     /* B, N or H < 1, or B*N*H*d > 2^31 - 2^16         */
    FA_ERR_HEADDIM = 3,   /* d is not 64 or 128                                 */
    FA_ERR_ALIGN = 4,     /* a pointer is not aligned as required               */
    FA_ERR_SCALE = 5,     /* softmax_scale is not finite                        */
    FA_ERR_WORKSPACE = 6, /* workspace missing or smaller than required         */
    FA_ERR_HIP = 7,       /* a HIP runtime call or kernel launch failed         */
    FA_ERR_DEVICE = 8,    /* the current device is not a gfx950 (MI355X) GPU    */
    FA_ERR_SCRATCH = 9    /* fa_decode_noalloc: the call needs more scratch than
                             the library's static scratch holds                 */
} fa_status;

/*
 * Forward pass: O = softmax(scale * Q K^T [+ causal mask]) V and its logsumexp.
 * (FlashAttention-2 abstract; IPLEX post, sections "Tiling preserves the
 * attention calculation" and "Three changes improve GPU utilisation".)
 *
 *   q, k, v   [B, N, H, d] bf16 inputs (read only)
 *   o         [B, N, H, d] bf16 output, rounded to nearest even
 *   lse       [B, H, N]    fp32 output, natural-log logsumexp (see above);
 *             it is what fa_bwd needs to recompute the probabilities
 */
FA_API fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int N, int H, int d, int causal, float softmax_scale,
                 hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for this problem size: two float32
 * [B, H, N] arrays (the row terms -D = -rowsum(dO * O) and L * log2(e)), each
 * starting on a 256-byte boundary. Returns 0 for an invalid shape.
 */
FA_API size_t fa_bwd_workspace_bytes(int B, int N, int H, int d);

/*
 * Backward pass of the forward above, recomputing the probabilities from the
 * saved logsumexp instead of storing them (the gradients must match within
 * tolerance: IPLEX post, section "Tiling preserves the attention
 * calculation"). With loss = sum(dO * O):
 *   D = rowsum(dO * O), dS = P * (dP - D) with dP = dO V^T,
 *   dV = P^T dO,  dQ = scale * dS K,  dK = scale * dS^T Q.
 *
 *   q, k, v      [B, N, H, d] bf16, the forward's inputs
 *   o, lse       the forward's outputs for the same inputs and flags
 *   dout         [B, N, H, d] bf16 upstream gradient dO
 *   dq, dk, dv   [B, N, H, d] bf16 outputs, rounded to nearest even
 *   workspace    device scratch of at least fa_bwd_workspace_bytes(B,N,H,d)
 *                bytes, 256-byte aligned, owned by the caller; its contents on
 *                entry do not matter and on return are unspecified. Two calls
 *                in flight at once need two workspaces.
 */
FA_API fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int B, int N, int H, int d, int causal, float softmax_scale,
                 hipStream_t stream);

/*
 * Attention of a query chunk over a key chunk: the unit of blockwise
 * attention in which a device keeps its queries and meets one key/value
 * block at a time (Ring Attention entry on the "High-Bandwidth Memory"
 * keyword page). Chunk results over disjoint key sets combine exactly with
 * fa_merge into the globally normalised result (IPLEX post, section "Tiling
 * preserves the attention calculation").
 *
 *   q          [B, Nq, H, d] bf16, query rows at global positions q_start ..
 *   k, v       [B, Nk, H, d] bf16, key rows at global positions k_start ..
 *   o          [B, Nq, H, d] float32 output: each row's attention output over
 *              the keys of this chunk it can see, normalised over those keys
 *              (16-byte aligned)
 *   lse        [B, H, Nq] float32 output: natural-log logsumexp over the same
 *              keys
 *   causal     key j is visible to query i iff k_start + j <= q_start + i;
 *              a row that sees no key of the chunk gets o = 0, lse = -inf.
 *              Non-causal: every key of the chunk is visible (the starts are
 *              then ignored).
 *   Nq >= 1, Nk >= 0 (Nk = 0 is an empty chunk: o = 0, lse = -inf, and k, v
 *   are not read). B*Nq*H*d and B*Nk*H*d must each be <= 2^31 - 2^16.
 *   Errors as for fa_fwd (FA_ERR_SHAPE also for Nq < 1 or Nk < 0).
 */
FA_API fa_status fa_fwd_chunk(const void* q, const void* k, const void* v, float* o, float* lse,
                       int B, int Nq, int Nk, int H, int d, int causal,
                       long long q_start, long long k_start, float softmax_scale,
                       hipStream_t stream);

/*
 * Exact combination of C chunk results over disjoint key sets (same
 * sources as fa_fwd_chunk):
 *   L = ln sum_c exp(L_c),   O = sum_c exp(L_c - L) O_c
 * Rows whose L_c is -inf in every chunk get O = 0 and L = -inf.
 *
 *   o_parts    [C, B, N, H, d] float32 (C fa_fwd_chunk outputs back to back),
 *              16-byte aligned
 *   lse_parts  [C, B, H, N] float32 (the matching logsumexp arrays)
 *   o          [B, N, H, d] bf16 output, rounded to nearest even
 *   lse        [B, H, N] float32 output, natural log
 *   1 <= C <= 65536; B, N, H >= 1; B*N*H*d <= 2^31 - 2^16; d = 64 or 128.
 *   FA_ERR_SHAPE for a C, B, N or H out of range.
 */
FA_API fa_status fa_merge(const float* o_parts, const float* lse_parts, int C, void* o, float* lse,
                   int B, int N, int H, int d, hipStream_t stream);

/*
 * Attention with an additive bias on the query-key scores (the bias abstract
 * on the related-papers page for "FlashAttention on a Napkin": prior
 * knowledge enters as a bias matrix added to the scores):
 *   S = scale * Q K^T + Bias  [+ causal mask],  O = softmax(S) V.
 *
 *   bias       bf16, element (b, h, i, j) at
 *              bias[b * bias_stride_b + h * bias_stride_h + i * bias_stride_row + j]
 *              (element strides; bias_stride_b or bias_stride_h may be 0 to
 *              share one matrix across batches or heads). bias_stride_row
 *              >= N and every stride a multiple of 8 (16-byte rows; pad the
 *              rows when N is not a multiple of 8), and every row, the last
 *              one included, spans bias_stride_row elements of readable
 *              device memory (a pitched [.., N, bias_stride_row] allocation);
 *              bias 16-byte aligned; (N + 64) * bias_stride_row * 2 < 2^32.
 *              Entries must be finite or -inf (-inf removes that key for
 *              that query); row padding may be read but never affects the
 *              result.
 *   o, lse     as for fa_fwd; a row whose every score is -inf gets o = 0 and
 *              lse = -inf.
 *   Other arguments and errors as for fa_fwd (FA_ERR_SHAPE also for a bias
 *   layout outside the rules above, FA_ERR_ALIGN for a misaligned bias).
 */
FA_API fa_status fa_fwd_bias(const void* q, const void* k, const void* v, const void* bias,
                      long long bias_stride_b, long long bias_stride_h, int bias_stride_row,
                      void* o, float* lse, int B, int N, int H, int d, int causal,
                      float softmax_scale, hipStream_t stream);

/*
 * Backward of fa_fwd_bias (same loss as fa_bwd). Gradients as for fa_bwd,
 * with the probabilities recomputed including the bias, and
 *   dBias = dS = P * (dP - D)   (the bias enters S with unit weight).
 *
 *   bias, strides   exactly as passed to fa_fwd_bias
 *   o, lse          fa_fwd_bias's outputs for the same inputs and flags
 *   dbias           bf16 output [B, H, N, N] with row stride
 *                   dbias_stride_row (>= N, multiple of 8; 16-byte aligned):
 *                   element (b, h, i, j) at ((b*H + h)*N + i)*dbias_stride_row + j.
 *                   Every element with i, j < N is written (0 where the
 *                   causal mask or a -inf bias hides the key); row padding
 *                   is left untouched. dBias is per (batch, head): for a bias
 *                   shared across batches or heads the caller sums over
 *                   them. NULL: dBias is not computed.
 *   workspace       as for fa_bwd (fa_bwd_workspace_bytes bytes).
 */
FA_API fa_status fa_bwd_bias(const void* q, const void* k, const void* v, const void* bias,
                      long long bias_stride_b, long long bias_stride_h, int bias_stride_row,
                      const void* o, const float* lse, const void* dout, void* dq, void* dk,
                      void* dv, void* dbias, int dbias_stride_row, void* workspace,
                      size_t workspace_bytes, int B, int N, int H, int d, int causal,
                      float softmax_scale, hipStream_t stream);

/*
 * FP8 (e4m3) forward, d = 64 or 128 (low-precision attention on narrow-format
 * matrix units: an abstract on the related-papers page for "FlashAttention
 * on a Napkin"; here the MI355X FP8 matrix unit). Same result definition as
 * fa_fwd, computed on the values the codes stand for:
 *
 *   q, k, v      uint8 OCP FP8 E4M3 codes, [B, N, H, d], 16-byte aligned
 *                (codes 0x7F / 0xFF are NaN and must not occur)
 *   q_descale,   float32 [B, H] each: the value of code c of (batch b, head h)
 *   k_descale,   is descale[b * H + h] * e4m3(c)
 *   v_descale
 *   o            [B, N, H, d] bf16 output; lse [B, H, N] float32 (natural
 *                log of the scaled scores of the dequantized inputs)
 *
 * Inside the kernel both products run on the FP8 matrix unit and the
 * probabilities are rounded to e4m3 for the P V product (the row sums and the
 * logsumexp use their fp32 values). That rounding bounds the error of each
 * output element by about 2^-4 times the probability-weighted mean of |V| in
 * its column (plus 2^-14 per key for probabilities below 2^-10), a bound the
 * tests check element by element. Errors as for fa_fwd (FA_ERR_HEADDIM for
 * d other than 64 or 128).
 */
FA_API fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                     const float* k_descale, const float* v_descale, void* o, float* lse,
                     int B, int N, int H, int d, int causal, float softmax_scale,
                     hipStream_t stream);

/*
 * Microscaled FP8 forward (the same low-precision abstract on the Napkin
 * related-papers list, read for matrix units that scale small blocks of
 * narrow-format values): Q, K, V as OCP FP8 E4M3 codes, each block of 32
 * consecutive elements along the reduction dimension of the product it enters
 * sharing one scale 2^(e - 127) given as an E8M0 byte e (255 is NaN and is not
 * checked for). Computes exact attention (as fa_fwd) on the values
 * e4m3(code) * 2^(e - 127); the matrix instruction applies the scales.
 *
 *   q, k, v      [B, N, H, d] uint8 e4m3 codes (16-byte aligned), d = 64 or 128
 *   q_scale,     [B, N, H, d / 32] uint8 E8M0: block i covers d = 32 i .. 32 i + 31
 *   k_scale        of one token
 *   v_scale      [B, ceil(N / 32), H, d] uint8 E8M0: block t of column d covers
 *                tokens 32 t .. 32 t + 31 (the last block may be short)
 *   o            [B, N, H, d] bf16 output; lse [B, H, N] float32 (natural log
 *                of the scaled scores of the values the codes stand for)
 *
 * The probabilities are rounded to e4m3 for the P V product as in
 * fa_fwd_fp8, with the same per-element error bound. Errors as for
 * fa_fwd_fp8.
 */
FA_API fa_status fa_fwd_mxfp8(const void* q, const void* q_scale, const void* k, const void* k_scale,
                       const void* v, const void* v_scale, void* o, float* lse, int B, int N, int H, int d,
                       int causal, float softmax_scale, hipStream_t stream);

/*
 * Decode-shaped attention: a few new query rows against a long key/value
 * history. The IPLEX post (section "Document the implementation
 * difference") separates decoding from prefill as a workload with its own
 * bottleneck: here it is streaming K and V from memory, so the keys are
 * split into ranges processed in parallel and their results are combined
 * exactly as fa_merge does (Ring Attention entry on the "High-Bandwidth
 * Memory" keyword page; post section "Tiling preserves the attention
 * calculation").
 *
 *   q          [B, Nq, H, d] bf16: the last Nq positions of the sequence
 *   k, v       [B, Nk, H, d] bf16: the whole sequence's keys and values
 *   o          [B, Nq, H, d] bf16 output (rounded to nearest even)
 *   lse        [B, H, Nq] float32 output, natural log
 *   causal     query row i sits at position Nk - Nq + i and sees key j iff
 *              j <= Nk - Nq + i (bottom-right alignment); with Nq > Nk the
 *              first Nq - Nk rows see no key and get o = 0, lse = -inf.
 *              Non-causal: every key is visible.
 *   workspace  device scratch of fa_decode_workspace_bytes(B, Nq, Nk, H, d)
 *              bytes, 256-byte aligned, owned by the caller (may be NULL
 *              when that size is 0); contents on entry do not matter. Two
 *              calls in flight at once need two workspaces.
 *   Nq, Nk >= 1 (any Nq; 1 ... 32 is the shape this entry point is built
 *   for). Errors as for fa_fwd; FA_ERR_WORKSPACE for a missing or short
 *   workspace.
 */
FA_API size_t fa_decode_workspace_bytes(int B, int Nq, int Nk, int H, int d);
FA_API fa_status fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Nq, int Nk, int H, int d, int causal, float softmax_scale,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_decode without a workspace argument and without any allocation: for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). It computes exactly
 * what fa_decode computes, with the same kernels; the key-split partial
 * results go to a static device array of the library (32 MiB, held by every
 * device the library runs on from module load until the process ends)
 * instead of a caller-supplied workspace.
 *
 *   Arguments as for fa_decode, minus workspace and workspace_bytes.
 *   FA_ERR_SCRATCH when the call would need more than 32 MiB of scratch,
 *   i.e. fa_decode_workspace_bytes(B, Nq, Nk, H, d) > 32 MiB (nothing is
 *   launched; fa_decode with a workspace handles such calls). Other errors
 *   as for fa_decode. The library calls no hipMalloc, hipFree or other
 *   allocating routine here.
 *   Every call on one device shares that device's scratch: calls that may
 *   overlap on one device (on different streams, or from several host
 *   threads without ordering) race on it and must not be issued.
 */
FA_API fa_status fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Nq, int Nk, int H, int d, int causal, float softmax_scale,
                            hipStream_t stream);

/* Human-readable text of a status code (a static string; never NULL). */
FA_API const char* fa_status_string(fa_status status);

/* Library version as major*10000 + minor*100 + patch. */
FA_API int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
