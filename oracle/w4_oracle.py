"""Oracle: the plain CPU definition of group-wise 4-bit weight-only quantization
(quantize, pack, unpack, dequantize), of the W4A16 linear
``y = x . dequant(W)^T + b`` and its input gradient, and of the LoRA merge
(dequantize, add a low-rank update, quantize again).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg import this module.  The HIP library never imports it, and the
two share no code, tables or constants.

Sources, cited by page and section:
  [LoopQ]  LoopQ ``packed_weight.py`` page: ``PackedLoopQWeight.validate``,
           ``payload_bytes``, ``_dequantize_validated``, ``state_dict``,
           ``pack_weight``.
  [Keras]  keras-nightly ``dense.py`` diff page: ``Dense._int4_build``,
           ``Dense._int4_call``, the int4 branch of ``Dense.quantize``.
  [Gemma]  Gemma peft ``_quantization_utils.py`` page: ``uniform_quantize``.
  [Paddle] PaddleNLP ``quantization_linear.py`` page: ``quant_weight_forward``,
           ``QuantizationLinearFunc``.
  [MAX]    Modular MAX ``graph/quantization.py`` page: ``QuantizationConfig``,
           ``QuantizationEncoding`` block parameters.

Arithmetic.  The codec runs in fp32: ``np.float32`` arrays and constants only,
IEEE round-to-nearest-even division, ``np.rint`` (round half to even).  The
linear runs in fp64.  bf16 values travel as ``uint16`` bit patterns.

Readings taken where the pages leave a step open:
  R1  Scales multiply: ``dq = v * s`` ([LoopQ] ``_dequantize_validated``).
  R2  Signed codes: the quantizer emits [-7, 7]; the decoder maps nibble
      values >= 8 to value - 16, so the reserved code 8 reads as -8
      ([LoopQ] ``validate``, format versions 1 and 2).
  R3  Symmetric group scale ``s = fp32(amax / 7)``;
      ``q = clamp(rint(fp32(w / s)), -7, 7)``.
  R4  Asymmetric (zero-point) group: ``lo = min(0, min w)``,
      ``hi = max(0, max w)``, ``s = fp32(fp32(hi - lo) / 15)``,
      ``z = clamp(rint(fp32(-lo / s)), 0, 15)``,
      ``q = clamp(rint(fp32(w / s)) + z, 0, 15)``; decode ``v = q - z``.
      (The quantizer's body is not on the [Keras] page; only its name and
      output shapes are.)
  R5  A group whose computed scale is 0 (all zeros, or underflow) gets s = 1.
  R6  The group of column k is ``g_idx[k]`` when a g_idx is given, else
      ``k // G`` ([Keras] ``_int4_build``, the g_idx initializer).
  R7  The linear uses the bf16-rounded dequantized weight (the [Keras] forward
      casts the dequantized kernel to the compute dtype before the matmul),
      accumulates in fp64 and adds the bias in fp64.
  R8  Group size -1 is per-channel: one group (one scale, and one zero-point
      in asym mode) per row, as the [Keras] block size -1 keeps one scale per
      output unit; any G >= K gives the same single group.
  R9  LoRA merge: the float domain is fp32 (the [Keras] merge adds the update
      to the dequantized kernel in the compute dtype; fp32 here).  The
      low-rank product is accumulated in fp64 in rank order and rounded once
      to fp32 (the page leaves the matmul's order to the backend); the merged
      weight is quantized again with the layer's group size, mode and g_idx.
  R10 Packed zero-points: the zero-points are 4-bit values, stored two per
      byte with the codes' nibble order (group 2j low, 2j+1 high).
  R11 GGUF Q4_0.  [MAX] fixes only the block: 32 weights in 2 + 16 bytes,
      the scale d then the 4-bit codes.  Everything else is a reading, not
      the page: d is fp16 (2 bytes, little-endian); codes are stored as
      q + 8 and read as (q - 8) * d; weight i of a block sits in the low
      nibble of byte i for i < 16 and in the high nibble of byte i - 16
      otherwise; the quantizer is the signed group-32 rule R3 taken against
      the stored fp16 scale.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
SYM = "sym"     # signed two's-complement nibbles, no zero-point
ASYM = "asym"   # unsigned nibbles with a per-group zero-point

__all__ = [
    "SYM", "ASYM", "PER_CHANNEL", "n_groups", "group_of_columns", "bf16_bits_to_f32",
    "f32_to_bf16_bits", "quantize", "pack_nibbles", "unpack_nibbles",
    "decode", "dequantize", "quantize_pack", "linear", "linear_grad_input", "validate_packed",
    "payload_bytes", "lora_merged_weight", "lora_merge", "pack_zeros", "unpack_zeros", "Q4_0_BLOCK", "Q4_0_BYTES",
    "q4_0_quantize", "q4_0_dequantize",
]


# ---------------------------------------------------------------------------
# shapes and groups
# ---------------------------------------------------------------------------
PER_CHANNEL = -1   # group size meaning one group per row (R8)


def n_groups(K: int, G: int) -> int:
    """Groups per row, ``ceil(K / G)`` ([Keras] ``_int4_build`` n_groups;
    [LoopQ] ``validate`` scale shape with G = 32); 1 for ``G = -1``, the
    per-channel block size of [Keras] ``_int4_build`` (R8)."""
    if G == PER_CHANNEL:
        return 1
    if G < 1:
        raise ValueError("G must be >= 1 or -1 (per-channel)")
    return -(-K // G)


def group_of_columns(K: int, G: int, g_idx=None) -> np.ndarray:
    """Group id of every input column (R6).  Default: contiguous blocks of G
    columns ([Keras] ``_int4_build``: floor of arange(input_dim) / block_size)."""
    if g_idx is None:
        if G == PER_CHANNEL:
            return np.zeros(K, dtype=np.int64)
        return np.arange(K, dtype=np.int64) // G
    gid = np.asarray(g_idx).astype(np.int64)
    if gid.shape != (K,):
        raise ValueError("g_idx must have one entry per input column")
    if gid.size and (gid.min() < 0 or gid.max() >= n_groups(K, G)):
        raise ValueError("g_idx entries must lie in [0, ceil(K/G))")
    return gid


# ---------------------------------------------------------------------------
# bf16 <-> fp32 (R7, [LoopQ] ``_dequantize_validated`` final ``.to(dtype)``)
# ---------------------------------------------------------------------------
def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening: a bf16 value is the top 16 bits of an fp32."""
    b = np.asarray(bits).astype(np.uint16)
    return (b.astype(np.uint32) << 16).view(F32)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Nearest bf16 to each finite fp32 value, ties to the even significand.

    Written as the definition: the two bf16 neighbours are the fp32 value
    truncated to 16 bits (toward zero) and the next bf16 away from zero; pick
    the nearer one, and on a tie the one whose last significand bit is 0.
    Distances are exact in fp64.  As IEEE 754 rounds as if the exponent range
    were unbounded, the neighbour past the largest finite bf16 counts as
    2^128 and a value rounding to it becomes infinity.
    """
    x = np.ascontiguousarray(x, dtype=F32)
    u = x.view(np.uint32)
    toward_zero = (u & np.uint32(0xFFFF0000)).astype(np.uint32)
    away = (toward_zero + np.uint32(0x10000)).astype(np.uint32)
    mag = np.abs(x.astype(np.float64))
    lo = np.abs(toward_zero.view(F32).astype(np.float64))
    with np.errstate(over="ignore", invalid="ignore"):
        hi = np.abs(away.view(F32).astype(np.float64))
        hi = np.where(np.isinf(hi), 2.0 ** 128, hi)
        d_lo = mag - lo
        d_hi = hi - mag
    even_lo = ((toward_zero >> np.uint32(16)) & np.uint32(1)) == 0
    pick_away = (d_hi < d_lo) | ((d_hi == d_lo) & ~even_lo)
    out = np.where(pick_away, away, toward_zero) >> np.uint32(16)
    return out.astype(np.uint16)


# ---------------------------------------------------------------------------
# quantize (R3, R4, R5)
# ---------------------------------------------------------------------------
def quantize(w, G: int, mode: str, g_idx=None):
    """Group-wise int4 quantization of ``w`` [N, K] (fp32 values).

    Returns ``(q, scales, zeros)``: ``q`` int16 [N, K] holding the integer
    codes (sym: [-7, 7]; asym: [0, 15]), ``scales`` fp32 [N, ceil(K/G)] and
    ``zeros`` uint8 [N, ceil(K/G)] (asym) or ``None`` (sym).

    Group statistics run over the member columns {k : gid(k) = g}; a group that
    no column maps to keeps s = 1 and z = 0 (R5).  Sym follows the absmax rule
    scale = max|w| / 7 with round half to even ([Gemma] ``uniform_quantize``
    uses the same rounding; [LoopQ] v1 forbids code -8, so the range is
    [-7, 7]).  Asym follows R4.
    """
    w = np.asarray(w, dtype=F32)
    if w.ndim != 2:
        raise ValueError("w must be a matrix")
    N, K = w.shape
    if mode not in (SYM, ASYM):
        raise ValueError("mode must be 'sym' or 'asym'")
    NG = n_groups(K, G)
    gid = group_of_columns(K, G, g_idx)
    q = np.zeros((N, K), dtype=np.int16)
    scales = np.ones((N, NG), dtype=F32)
    zeros = np.zeros((N, NG), dtype=np.uint8) if mode == ASYM else None
    for g in range(NG):
        cols = np.nonzero(gid == g)[0]
        if cols.size == 0:
            continue
        blk = w[:, cols]
        if mode == SYM:
            amax = np.max(np.abs(blk), axis=1)
            s = (amax / F32(7)).astype(F32)
            s[s == F32(0)] = F32(1)
            r = np.rint((blk / s[:, None]).astype(F32))
            q[:, cols] = np.clip(r, -7, 7).astype(np.int16)
        else:
            lo = np.minimum(np.min(blk, axis=1), F32(0))
            hi = np.maximum(np.max(blk, axis=1), F32(0))
            span = (hi - lo).astype(F32)
            s = (span / F32(15)).astype(F32)
            s[s == F32(0)] = F32(1)
            z = np.clip(np.rint((-lo / s).astype(F32)), 0, 15)
            r = np.rint((blk / s[:, None]).astype(F32))
            q[:, cols] = np.clip(r + z[:, None], 0, 15).astype(np.int16)
            zeros[:, g] = z.astype(np.uint8)
        scales[:, g] = s
    return q, scales, zeros


# ---------------------------------------------------------------------------
# pack / unpack ([LoopQ] ``pack_weight``, ``_dequantize_validated``)
# ---------------------------------------------------------------------------
def pack_nibbles(q) -> np.ndarray:
    """Two codes per byte along the row ([LoopQ] ``pack_weight``, nibble
    order 'even_column_low'; the format, not the listing): a code's nibble is
    its 4-bit two's-complement pattern (q & 15); byte j of a row holds column
    2j in bits 0..3 and column 2j+1 in bits 4..7; when K is odd the last
    byte's bits 4..7 are 0.  Written byte by byte."""
    q = np.asarray(q)
    N, K = q.shape
    nib_t = np.ascontiguousarray((q.astype(np.int16) & 15).astype(np.uint8).T)   # [K, N]: column k of every row
    out_t = np.zeros(((K + 1) // 2, N), dtype=np.uint8)                           # [byte j, row]
    for j in range(out_t.shape[0]):
        low = nib_t[2 * j]
        high = nib_t[2 * j + 1] if 2 * j + 1 < K else np.zeros(N, np.uint8)
        out_t[j] = low | (high << np.uint8(4))
    return np.ascontiguousarray(out_t.T)


def unpack_nibbles(codes, K: int) -> np.ndarray:
    """Inverse of ``pack_nibbles``: uint8 [N, K] nibble values 0..15; column
    k is bits 0..3 of byte k // 2 for even k and bits 4..7 for odd k
    ([LoopQ] ``_dequantize_validated``)."""
    c_t = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8).T)   # [byte j, row]
    N = c_t.shape[1]
    out_t = np.zeros((K, N), dtype=np.uint8)                          # [column k, row]
    for k in range(K):
        byte = c_t[k // 2]
        out_t[k] = (byte >> np.uint8(4)) if k % 2 else (byte & np.uint8(15))
    return np.ascontiguousarray(out_t.T)


def decode(u, mode: str, zeros=None, gid=None) -> np.ndarray:
    """Integer value of each nibble.  Sym: 4-bit two's complement, bit 3
    weighs -8 and bits 0..2 weigh 4, 2, 1 ([LoopQ] ``_dequantize_validated``:
    values from 8 up read as negative).  Asym: v = u - z[n, gid(k)] (R4),
    exact in integers."""
    u = np.asarray(u).astype(np.int32)
    if mode == SYM:
        return -8 * ((u >> 3) & 1) + (u & 7)
    return u - np.asarray(zeros).astype(np.int32)[:, gid]


def dequantize(codes, scales, zeros, g_idx, K: int, G: int, mode: str,
               out: str = "bf16") -> np.ndarray:
    """Dense weight from packed codes: ``d = fp32(v) * s[n, gid(k)]`` (one
    fp32 multiply), then cast ([LoopQ] ``_dequantize_validated``; [Keras]
    ``_int4_call`` dequantize-with-scale/zero map).  ``out='bf16'`` returns
    uint16 bit patterns (R7), ``out='f32'`` the fp32 values."""
    gid = group_of_columns(K, G, g_idx)
    v = decode(unpack_nibbles(codes, K), mode, zeros, gid)
    s = np.asarray(scales, dtype=F32)[:, gid]
    d = (v.astype(F32) * s).astype(F32)
    if out == "f32":
        return d
    if out == "bf16":
        return f32_to_bf16_bits(d)
    raise ValueError("out must be 'bf16' or 'f32'")


def quantize_pack(w, G: int, mode: str, g_idx=None):
    """quantize then pack: ``(codes uint8 [N, ceil(K/2)], scales, zeros)``
    ([LoopQ] ``pack_weight``; [Keras] ``quantize`` int4 branch)."""
    q, scales, zeros = quantize(w, G, mode, g_idx)
    return pack_nibbles(q), scales, zeros


# ---------------------------------------------------------------------------
# linear ([Keras] ``_int4_call``; [Paddle] ``quant_weight_forward``)
# ---------------------------------------------------------------------------
def linear(x_bits, codes, scales, zeros, g_idx, K: int, G: int, mode: str,
           bias_bits=None, row_chunk: int = 4096) -> np.ndarray:
    """``y[m, n] = sum_k x[m, k] * Wd[n, k] + b[n]`` in fp64, where Wd is the
    bf16-rounded dequantized weight (R7).  ``x_bits`` uint16 [M, K] and
    ``bias_bits`` uint16 [N] are bf16 bit patterns.  Returns fp64 [M, N].
    Rows of W are processed in chunks only to bound memory."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    codes = np.asarray(codes)
    N = codes.shape[0]
    y = np.empty((x.shape[0], N), dtype=np.float64)
    for n0 in range(0, N, row_chunk):
        n1 = min(N, n0 + row_chunk)
        z = None if zeros is None else np.asarray(zeros)[n0:n1]
        wd = bf16_bits_to_f32(dequantize(codes[n0:n1], np.asarray(scales)[n0:n1],
                                         z, g_idx, K, G, mode, "bf16"))
        y[:, n0:n1] = x @ wd.astype(np.float64).T
    if bias_bits is not None:
        y += bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    return y


def linear_grad_input(dy_bits, codes, scales, zeros, g_idx, K: int, G: int, mode: str,
                      row_chunk: int = 4096) -> np.ndarray:
    """Input gradient of the linear: ``dx[m, k] = sum_n dy[m, n] * Wd[n, k]``
    in fp64, with the same bf16-rounded dequantized weight Wd as the forward
    (R7).  ([Keras] the custom gradient of the sub-channel int4 matmul: the
    upstream gradient times the dequantized kernel cast to the compute dtype;
    [Paddle] ``QuantizationLinearFunc`` backward: the output gradient times
    the dequantized weight.)  ``dy_bits`` uint16 [M, N] bf16 bit patterns.
    Returns fp64 [M, K]."""
    dy = bf16_bits_to_f32(dy_bits).astype(np.float64)
    codes = np.asarray(codes)
    N = codes.shape[0]
    dx = np.zeros((dy.shape[0], K), dtype=np.float64)
    for n0 in range(0, N, row_chunk):
        n1 = min(N, n0 + row_chunk)
        z = None if zeros is None else np.asarray(zeros)[n0:n1]
        wd = bf16_bits_to_f32(dequantize(codes[n0:n1], np.asarray(scales)[n0:n1],
                                         z, g_idx, K, G, mode, "bf16"))
        dx += dy[:, n0:n1] @ wd.astype(np.float64)
    return dx


# ---------------------------------------------------------------------------
# format checks ([LoopQ] ``validate``, ``payload_bytes``)
# ---------------------------------------------------------------------------
# ---------------------------------------------------------------------------
# packed zero-points (R10)
# ---------------------------------------------------------------------------
def pack_zeros(zeros) -> np.ndarray:
    """Zero-points two per byte along the row, group 2j in the low nibble of
    byte j and group 2j+1 in the high nibble (the [LoopQ] nibble order of the
    codes); an odd group count leaves the last high nibble 0.  uint8 [N, NG]
    -> uint8 [N, ceil(NG/2)]."""
    z = np.asarray(zeros)
    if z.ndim != 2 or z.size and (z.min() < 0 or z.max() > 15):
        raise ValueError("zeros must be a matrix of values 0..15")
    return pack_nibbles(z.astype(np.int16))


def unpack_zeros(packed, NG: int) -> np.ndarray:
    """Inverse of ``pack_zeros``: uint8 [N, ceil(NG/2)] -> uint8 [N, NG]."""
    return unpack_nibbles(packed, NG).astype(np.uint8)


# ---------------------------------------------------------------------------
# GGUF Q4_0 block codec (R11)
# ---------------------------------------------------------------------------
Q4_0_BLOCK = 32    # weights per block ([MAX] block parameters of Q4_0)
Q4_0_BYTES = 18    # the block's 2-byte scale d, then 16 bytes of 4-bit codes


def q4_0_quantize(w) -> np.ndarray:
    """Quantize ``w`` fp32 [N, K] (K a multiple of 32) into Q4_0 blocks,
    uint8 [N, K/32, 18] (R11): per block of 32 consecutive weights of a row
    ``d = fp16(fp32(amax / 7))``; ``q = clamp(rint(fp32(w / d)), -7, 7)``
    with d widened back to fp32 (every code 0 when d is 0); bytes 0..1 hold d
    (little-endian fp16), byte 2 + i holds q[i] + 8 in its low nibble and
    q[i + 16] + 8 in its high nibble."""
    w = np.asarray(w, dtype=F32)
    N, K = w.shape
    if K % Q4_0_BLOCK:
        raise ValueError("Q4_0 needs K to be a multiple of 32")
    nb = K // Q4_0_BLOCK
    blk = w.reshape(N, nb, Q4_0_BLOCK)
    amax = np.max(np.abs(blk), axis=2)
    d16 = (amax / F32(7)).astype(F32).astype(np.float16)
    d = d16.astype(F32)
    safe = np.where(d == F32(0), F32(1), d)
    q = np.clip(np.rint((blk / safe[..., None]).astype(F32)), -7, 7)
    q = np.where(d[..., None] == F32(0), 0, q)
    u = (q + 8).astype(np.uint8)
    out = np.empty((N, nb, Q4_0_BYTES), dtype=np.uint8)
    out[..., 0:2] = d16.astype("<f2").view(np.uint8).reshape(N, nb, 2)
    out[..., 2:] = u[..., :16] | (u[..., 16:] << 4)
    return out


def q4_0_dequantize(blocks, out: str = "f32") -> np.ndarray:
    """Dense weight [N, 32 * nb] from Q4_0 blocks uint8 [N, nb, 18]:
    ``fp32(q - 8) * d`` (one fp32 multiply), ``out='bf16'`` gives the RNE
    bf16 bit patterns."""
    b = np.asarray(blocks, dtype=np.uint8)
    N, nb, _ = b.shape
    d = np.ascontiguousarray(b[..., 0:2]).view("<f2")[..., 0].astype(F32)
    qs = b[..., 2:]
    u = np.concatenate([qs & 15, qs >> 4], axis=-1).astype(np.int16)
    v = ((u - 8).astype(F32) * d[..., None]).astype(F32).reshape(N, nb * Q4_0_BLOCK)
    return f32_to_bf16_bits(v) if out == "bf16" else v


# ---------------------------------------------------------------------------
# LoRA merge ([Keras] ``Dense._get_kernel_with_merged_lora``)
# ---------------------------------------------------------------------------
def lora_merged_weight(codes, scales, zeros, g_idx, K: int, G: int, mode: str,
                       lora_a, lora_b, lora_scale: float) -> np.ndarray:
    """The float-domain merge, fp32 [N, K]:
    ``Wd[n, k] + c * AB[n, k]`` with ``AB[n, k] = sum_j A[k, j] B[j, n]``.

    ``lora_a`` fp32 [K, r] and ``lora_b`` fp32 [r, N] as the [Keras] layer
    stores them (input features x rank, rank x units), ``c = fp32(lora_scale)``
    (alpha / rank).  Steps (R9): Wd is the fp32 dequantized weight; AB is
    accumulated in fp64 over j = 0 .. r-1 in that order (every product of two
    fp32 values is exact in fp64) and rounded once to fp32; then
    ``delta = fp32(c * AB)`` and ``merged = fp32(Wd + delta)``.
    """
    wd = dequantize(codes, scales, zeros, g_idx, K, G, mode, out="f32")
    A = np.asarray(lora_a, dtype=F32)
    B = np.asarray(lora_b, dtype=F32)
    N = wd.shape[0]
    if A.ndim != 2 or A.shape[0] != K or B.shape != (A.shape[1], N):
        raise ValueError("lora_a must be [K, r] and lora_b [r, N]")
    acc = np.zeros((N, K), dtype=np.float64)
    for j in range(A.shape[1]):
        acc += B[j].astype(np.float64)[:, None] * A[:, j].astype(np.float64)[None, :]
    delta = (F32(lora_scale) * acc.astype(F32)).astype(F32)
    return (wd + delta).astype(F32)


def lora_merge(codes, scales, zeros, g_idx, K: int, G: int, mode: str,
               lora_a, lora_b, lora_scale: float):
    """Merge a low-rank update into a packed weight and quantize the result
    again with the same group size, mode and group map ([Keras]
    ``Dense._get_kernel_with_merged_lora``: dequantize, add
    ``(alpha / rank) * A B``, re-quantize and pack).  Returns
    ``(codes, scales, zeros)`` of the merged weight."""
    merged = lora_merged_weight(codes, scales, zeros, g_idx, K, G, mode, lora_a, lora_b, lora_scale)
    return quantize_pack(merged, G, mode, g_idx)


def validate_packed(codes, scales, zeros, K: int, G: int, mode: str,
                    g_idx=None, narrow: bool = True) -> None:
    """Raise ValueError unless the packed tensors satisfy the format rules:
    codes uint8 [N, ceil(K/2)]; scales fp32 [N, ceil(K/G)], finite and > 0;
    zeros uint8 with the scales' shape and values <= 15 (asym); a 0 high
    nibble in the last byte when K is odd; with ``narrow`` (LoopQ format v1),
    no signed code 8 (-8)."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    if codes.dtype != np.uint8 or codes.ndim != 2 or codes.shape[1] != -(-K // 2):
        raise ValueError("packed code shape/dtype mismatch")
    N = codes.shape[0]
    if scales.dtype != F32 or scales.shape != (N, n_groups(K, G)):
        raise ValueError("scale shape/dtype mismatch")
    if not np.all(np.isfinite(scales)) or not np.all(scales > 0):
        raise ValueError("scales must be finite and positive")
    if K % 2 and np.any(codes[:, -1] >> 4):
        raise ValueError("nonzero unused high nibble")
    if mode == ASYM:
        zeros = np.asarray(zeros)
        if zeros.dtype != np.uint8 or zeros.shape != scales.shape or np.any(zeros > 15):
            raise ValueError("zero-point shape/dtype/range mismatch")
    elif zeros is not None:
        raise ValueError("symmetric codes carry no zero-points")
    elif narrow:
        u = unpack_nibbles(codes, K)
        if np.any(u == 8):
            raise ValueError("code -8 is outside the narrow signed range")
    group_of_columns(K, G, g_idx)


def payload_bytes(codes, scales, zeros=None) -> int:
    """Tensor payload only: code bytes + 4 bytes per scale (+ 1 byte per
    zero-point) ([LoopQ] ``payload_bytes``)."""
    n = int(np.asarray(codes).size) + 4 * int(np.asarray(scales).size)
    if zeros is not None:
        n += int(np.asarray(zeros).size)
    return n
