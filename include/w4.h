/*
 * w4.h — C ABI of libw4.so: group-wise 4-bit weight-only quantization and the
 * W4A16 linear  y = x . dequant(W)^T + b  on AMD MI355X (gfx950).
 *
 * Data format (shared by every entry point)
 * -----------------------------------------
 *   W       [N, K]  the dense weight (N output features, K input features).
 *   codes   uint8 [N, ceil(K/2)], row-major.  Two 4-bit codes per byte along a
 *           row: column 2j in the low nibble of byte j, column 2j+1 in the high
 *           nibble; when K is odd the unused high nibble of each row's last
 *           byte is 0.  (LoopQ packed_weight.py page: pack_weight, validate,
 *           nibble order 'even_column_low'.)
 *   scales  fp32 [N, ceil(K/G)], row-major: one multiplicative scale per row
 *           and group (same page: _dequantize_validated multiplies).
 *   zeros   uint8 [N, ceil(K/G)] zero-points 0..15, one per byte (W4_ASYM;
 *           the keras dense.py diff page stores a kernel_zero per group), or
 *           uint8 [N, ceil(ceil(K/G)/2)] two per byte (W4_ASYM_PACKED).
 *   G       group size: a multiple of 8 (>= 8), or per-channel, one group per
 *           row, given as W4_PER_CHANNEL (-1) or any G >= K (keras dense.py
 *           diff page: block size -1, one scale per output unit).  Below,
 *           ceil(K/G) reads 1 for per-channel.
 *   g_idx   int32 [K] group of each input column, values in [0, ceil(K/G));
 *           NULL means column k belongs to group k / G (keras dense.py diff
 *           page: _int4_build g_idx initializer; MAX quantization.py page:
 *           desc_act, activation order).
 *
 * Code modes
 *   W4_SYM   signed two's-complement nibbles: nibble c means c - 16 when c >= 8
 *            (LoopQ page, _dequantize_validated).  The quantizer emits
 *            [-7, 7]: scale = max|w| / 7 over the group.  Decoding accepts -8.
 *   W4_ASYM  unsigned nibbles with a per-group zero-point z: value = c - z.
 *            Quantizer: lo = min(0, min w), hi = max(0, max w),
 *            s = (hi - lo) / 15, z = clamp(rint(-lo / s), 0, 15),
 *            c = clamp(rint(w / s) + z, 0, 15).
 *   W4_ASYM_PACKED  W4_ASYM with the zero-points stored two per byte:
 *            zeros uint8 [N, ceil(NG/2)], group 2j in the low nibble of byte
 *            j and group 2j+1 in the high nibble (the keras dense.py diff page
 *            keeps kernel_zero as 4-bit values; the nibble order is the codes'
 *            order of the LoopQ page; the layout w4_pack_zeros writes).
 *            Accepted wherever zero-points are read: w4_dequantize,
 *            w4_linear, w4_linear_noalloc, w4_linear_grad_input.
 *            w4_quantize_pack and w4_lora_merge write one zero-point per byte
 *            and return W4_ERR_UNSUPPORTED for this mode.
 *   Both: a group whose computed scale is 0 gets scale 1.  Divisions are IEEE
 *   fp32 round-to-nearest, rint rounds half to even.
 *
 * Conventions for every call
 *   - Pointers are device pointers (hipMalloc / PyTorch-ROCm allocations) on
 *     the current device, owned by the caller, dense row-major, 16-byte aligned
 *     base addresses.  The library keeps no reference after returning.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on it and return; they never synchronize.
 *   - Arguments are checked on the host before any launch.  On failure the
 *     call returns a non-zero status, writes nothing, and w4_last_error()
 *     describes the problem.  No C++ exception crosses this boundary.
 *   - Not checked (the caller's responsibility, as the LoopQ page's owner
 *     validates before use): finite weights, g_idx values in range, zeros
 *     <= 15, finite positive scales, a 0 pad nibble.  Violations give
 *     unspecified values but every access stays in bounds.
 */
#ifndef W4_H
#define W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4_ABI_VERSION 2

/* Group size meaning one group per row (per-channel scales). */
#define W4_PER_CHANNEL (-1)

typedef enum {
  W4_OK = 0,
  W4_ERR_INVALID_ARG = 1,  /* bad size, null pointer, misaligned pointer, mode */
  W4_ERR_UNSUPPORTED = 2,  /* valid request the library does not implement  */
  W4_ERR_HIP = 3           /* a HIP runtime call or kernel launch failed     */
} w4_status;

typedef enum { W4_F32 = 0, W4_BF16 = 1 } w4_dtype;
typedef enum { W4_SYM = 0, W4_ASYM = 1, W4_ASYM_PACKED = 2 } w4_mode;

/* Version of this ABI (W4_ABI_VERSION). */
int w4_abi_version(void);

/* Static text for a status code. */
const char* w4_status_string(int status);

/* Detail of the last failed call on this host thread ("" if none). */
const char* w4_last_error(void);

/*
 * w4_quantize_pack — quantize W group-wise and pack the codes.
 *   (LoopQ packed_weight.py page: pack_weight; keras dense.py diff page:
 *    Dense.quantize, int4 branch with block_size.)
 *   w        [N, K] finite weights, fp32 (w_dtype = W4_F32) or bf16 (W4_BF16);
 *            codes of non-finite weights are unspecified.
 *   N, K     >= 1 (an empty matrix is rejected, as pack_weight rejects it).
 *   G        group size (see Data format); at most 4096 groups per row,
 *            ceil(K/G) <= 4096 (else W4_ERR_UNSUPPORTED).
 *   mode     W4_SYM or W4_ASYM.
 *   g_idx    int32 [K] or NULL (contiguous groups).  Group statistics run over
 *            the columns mapped to each group; a group no column maps to gets
 *            scale 1 (and zero-point 0).
 *   codes    out uint8 [N, ceil(K/2)].
 *   scales   out fp32  [N, ceil(K/G)].
 *   zeros    out uint8 [N, ceil(K/G)] for W4_ASYM; must be NULL for W4_SYM.
 * Outputs are bit-exact functions of the inputs (no atomics on values).
 */
w4_status w4_quantize_pack(const void* w, int w_dtype, int64_t N, int64_t K,
                           int64_t G, int mode, const int32_t* g_idx,
                           uint8_t* codes, float* scales, uint8_t* zeros,
                           void* stream);

/*
 * w4_dequantize — dense weight from packed codes.
 *   (LoopQ packed_weight.py page: _dequantize_validated; keras dense.py diff
 *    page: dequantize with scale/zero map and g_idx; PaddleNLP
 *    quantization_linear.py page: weight_dequantize.)
 *   out[n, k] = fp32(value(n, k)) * scales[n, gid(k)]   (one fp32 multiply),
 *   stored as fp32 (out_dtype = W4_F32) or rounded to nearest-even bf16
 *   (W4_BF16).  Arguments as in w4_quantize_pack; out is [N, K].
 */
w4_status w4_dequantize(const uint8_t* codes, const float* scales,
                        const uint8_t* zeros, const int32_t* g_idx,
                        int64_t N, int64_t K, int64_t G, int mode,
                        void* out, int out_dtype, void* stream);

/*
 * w4_linear_workspace_bytes — device scratch w4_linear needs for this shape
 * (0 when none).  The prefill path (M > 16) stages the bf16 dequantized weight
 * [N, K] there; the batched decode path (4 < M <= 16) may split K over a few
 * workgroups and keep their fp32 partial sums there (splits * M * N * 4
 * bytes), then add them in a fixed order.
 */
size_t w4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G,
                                 int mode, int has_g_idx);

/*
 * w4_linear — W4A16 linear  y[m, n] = sum_k x[m, k] * Wd[n, k] + bias[n].
 *   (keras dense.py diff page: Dense._int4_call, sub-channel branch, then the
 *    bias add; PaddleNLP quantization_linear.py page: weight_only_linear with
 *    group_size.)
 *   x        bf16 [M, K] activations (not quantized: weight-only, A16).
 *   M        >= 0 (M = 0 returns W4_OK and launches nothing).
 *   codes, scales, zeros, g_idx, N, K, G, mode  as in w4_dequantize.
 *   bias     bf16 [N] or NULL.
 *   y        out bf16 [M, N]; products accumulate in fp32, the bias is added
 *            in fp32, one rounding to bf16 at the end.
 *   workspace, workspace_bytes  device scratch of at least
 *            w4_linear_workspace_bytes(...) bytes (may be NULL when that is 0).
 * Results are deterministic: the same inputs give the same bits.
 */
w4_status w4_linear(const void* x, int64_t M,
                    const uint8_t* codes, const float* scales,
                    const uint8_t* zeros, const int32_t* g_idx,
                    int64_t N, int64_t K, int64_t G, int mode,
                    const void* bias, void* y,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4_linear_noalloc — w4_linear for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same operation, arguments and results as w4_linear,
 * without the workspace.  Scratch the kernels need (the split-K partial sums
 * of the batched decode path, the staged weight of the prefill path) lives in
 * a fixed device array of w4_linear_noalloc_max_scratch_bytes() bytes that
 * every GPU the library runs on holds until the process ends; the call
 * allocates and frees nothing.  A shape whose w4_linear_workspace_bytes
 * exceeds that size returns W4_ERR_UNSUPPORTED and launches nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams, or from different host threads without ordering)
 * race on it.  No contents carry over from one call to the next.
 */
size_t w4_linear_noalloc_max_scratch_bytes(void);
w4_status w4_linear_noalloc(const void* x, int64_t M,
                            const uint8_t* codes, const float* scales,
                            const uint8_t* zeros, const int32_t* g_idx,
                            int64_t N, int64_t K, int64_t G, int mode,
                            const void* bias, void* y, void* stream);

/*
 * w4_linear_grad_input_workspace_bytes — device scratch w4_linear_grad_input
 * needs for this shape: fp32 partial sums of row slices for M <= 16, the
 * transposed bf16 dequantized weight [K, N] for M > 16.
 */
size_t w4_linear_grad_input_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G,
                                            int mode, int has_g_idx);

/*
 * w4_linear_grad_input — input gradient of w4_linear:
 *   dx[m, k] = sum_n dy[m, n] * Wd[n, k].
 *   (keras dense.py diff page: the custom gradient of the sub-channel int4
 *    matmul, the upstream gradient times the dequantized kernel cast to the
 *    compute dtype; PaddleNLP quantization_linear.py page:
 *    QuantizationLinearFunc.backward, the output gradient times the
 *    dequantized weight.)
 *   dy       bf16 [M, N] upstream gradient.
 *   M        >= 0 (M = 0 returns W4_OK and launches nothing).
 *   codes, scales, zeros, g_idx, N, K, G, mode  as in w4_linear.
 *   dx       out bf16 [M, K]; products accumulate in fp32 in a fixed order
 *            (the same inputs give the same bits), one rounding to bf16.
 *   workspace, workspace_bytes  device scratch of at least
 *            w4_linear_grad_input_workspace_bytes(...) bytes (never NULL).
 */
w4_status w4_linear_grad_input(const void* dy, int64_t M,
                               const uint8_t* codes, const float* scales,
                               const uint8_t* zeros, const int32_t* g_idx,
                               int64_t N, int64_t K, int64_t G, int mode,
                               void* dx, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * w4_lora_merge_workspace_bytes — device scratch w4_lora_merge needs: 0 when
 * the merge runs in one pass (no g_idx, G a power of two in [8, 512]), else
 * the merged fp32 weight, N * K * 4 bytes.
 */
size_t w4_lora_merge_workspace_bytes(int64_t N, int64_t K, int64_t G, int mode,
                                     int has_g_idx, int64_t rank);

/*
 * w4_lora_merge — fold a low-rank (LoRA) update into a packed weight and
 * quantize the sum again.
 *   (keras dense.py diff page: Dense._get_kernel_with_merged_lora —
 *    dequantize, add (lora_alpha / lora_rank) * lora_kernel_a @ lora_kernel_b
 *    in the float domain, re-quantize with the layer's block size, pack.)
 *   merged[n, k] = fp32( fp32(v[n, k] * s[n, gid(k)])
 *                        + fp32(lora_scale * fp32(sum_j A[k, j] * B[j, n])) )
 *   The rank sum is accumulated in fp64 in order j = 0 .. rank-1 (each product
 *   of two fp32 values is exact there) and rounded once to fp32.  The merged
 *   weight is then quantized exactly as w4_quantize_pack quantizes an fp32
 *   weight with the same G, mode and g_idx.
 *   codes, scales, zeros, g_idx, N, K, G, mode  the packed weight, as in
 *            w4_dequantize; at most 4096 groups per row.
 *   lora_a   fp32 [K, rank] (input features x rank).
 *   lora_b   fp32 [rank, N] (rank x output features).
 *   rank     1 <= rank <= 64 (larger: W4_ERR_UNSUPPORTED).
 *   lora_scale  the update's factor, alpha / rank.
 *   codes_out, scales_out, zeros_out  out, shaped as codes, scales, zeros
 *            (zeros_out NULL for W4_SYM).  Each may be the same pointer as
 *            its input (merge in place); otherwise outputs must not overlap
 *            the inputs.
 *   workspace, workspace_bytes  device scratch of at least
 *            w4_lora_merge_workspace_bytes(...) bytes (may be NULL when 0).
 * Outputs are bit-exact functions of the inputs.
 */
w4_status w4_lora_merge(const uint8_t* codes, const float* scales,
                        const uint8_t* zeros, const int32_t* g_idx,
                        int64_t N, int64_t K, int64_t G, int mode,
                        const float* lora_a, const float* lora_b, int64_t rank,
                        float lora_scale,
                        uint8_t* codes_out, float* scales_out, uint8_t* zeros_out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4_pack_zeros / w4_unpack_zeros — zero-points in the compact 4-bit storage:
 * packed uint8 [N, ceil(NG/2)], group 2j in the low nibble of byte j and
 * group 2j+1 in the high nibble (the codes' nibble order, LoopQ
 * packed_weight.py page; the keras dense.py diff page keeps one zero-point
 * per group); an odd NG leaves the last high nibble 0.  The compute entry
 * points take the unpacked form, uint8 [N, NG].
 *   zeros    uint8 [N, NG], values 0..15 (only the low nibble is packed).
 *   N, NG    >= 1.
 *   packed   uint8 [N, ceil(NG/2)].
 * No alignment requirement.
 */
w4_status w4_pack_zeros(const uint8_t* zeros, int64_t N, int64_t NG, uint8_t* packed, void* stream);
w4_status w4_unpack_zeros(const uint8_t* packed, int64_t N, int64_t NG, uint8_t* zeros, void* stream);

/*
 * w4_q4_0_quantize / w4_q4_0_dequantize — Q4_0 blocks
 * (Modular MAX quantization.py page: QuantizationEncoding Q4_0, 32 weights
 * per block in 2 + 16 bytes, the scale d then the 4-bit codes).  The page
 * fixes only that block size and byte count; the fp16 d, the +8 offset, the
 * nibble placement and the quantizer below are this library's reading.
 *   Block layout: bytes 0..1 the fp16 scale d (little-endian); byte 2 + i
 *   holds q[i] + 8 in its low nibble and q[i + 16] + 8 in its high nibble;
 *   weight i of the block reads as fp32(q[i] - 8) * d.
 *   Quantizer: d = fp16(fp32(max |w| / 7)) over the block (nearest, ties to
 *   even), q = clamp(rint(fp32(w / d)), -7, 7) with d widened to fp32, all
 *   codes 0 when d is 0 — the signed group rule of w4_quantize_pack taken
 *   against the stored fp16 scale.  Weights must be finite with
 *   max |w| / 7 within fp16 range (else the block is unspecified).
 *   w        [N, K] fp32 (W4_F32) or bf16 (W4_BF16), 16-byte aligned.
 *   N, K     N >= 1, K a positive multiple of 32.
 *   blocks   uint8 [N, K/32, 18] (18 * N * K / 32 bytes), 16-byte aligned.
 *   out      [N, K] fp32 or bf16 (RNE), 16-byte aligned.
 */
w4_status w4_q4_0_quantize(const void* w, int w_dtype, int64_t N, int64_t K, uint8_t* blocks, void* stream);
w4_status w4_q4_0_dequantize(const uint8_t* blocks, int64_t N, int64_t K, void* out, int out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4_H */
