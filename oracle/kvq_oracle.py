"""CPU oracle for the rotated INT2 KV cache: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the entry point's smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code, tables or
constants with the HIP library; the two meet only through the documented
cache layout and the seeded input generators.

What it computes, and where that comes from:

* A per-head orthogonal rotation R is applied to K and V rows before 2-bit
  quantization and is removed from the attention output afterwards
  ("Output-Aware Rotation for INT2 KV-Cache Quantization", woor.ai page,
  section "Key Details", second bullet; the readout is the scaled
  dot-product attention named in "What You Need to Know").
* The rotation is either a normalized Walsh-Hadamard matrix, whose fast
  transform is the efficient form (RotateKV, IJCAI 2025 record, abstract
  item (i); KVLinC, fugumt page, abstract: "Hadamard rotation"), or a dense
  learned per-head orthogonal matrix (OptR, same woor.ai page, "What You
  Need to Know").
* The codec: asymmetric 2-bit codes in channel groups of 32 with an fp16
  scale and an fp16 zero-point (the group minimum), four codes per byte.
  The pages name INT2 but fix none of these parameters; they are this
  library's format, and every step below that the pages leave open is a
  stated reading (listed in the design notes).
* Other bit widths: the same codec with b = 1 or 4 bits per code
  (2**b - 1 levels above the zero-point, 8/b codes per byte), so that keys
  and values can be kept at different widths.  The pages name mixed-bit
  schemes and binary codes as directions only (OptR page, the future-work
  paragraph and "Why It Matters"; the mixed-precision entries of the
  related-work list) and fix nothing about them; b = 2 is the INT2 codec.

Precision: the rotation and the attention are evaluated in fp64.  The
quantizer is a fixed sequence of IEEE binary32 operations (subtract,
divide, multiply, round-half-even) followed by RNE conversion to fp16;
numpy float32 arithmetic performs exactly those operations, so they are
written in float32 here.  No fused multiply-add is used anywhere.

Cache layout (the library's boundary format, [B][Hkv][T_cap][...]):
    codes  uint8   [..., d/4]  channel 4*b+i in bits 2i..2i+1 of byte b
                   (b-bit codes: [..., d*b/8], channel (8/b)*j+i in bits
                   b*i .. b*i+b-1 of byte j)
    scales float16 [..., d/group]
    zeros  float16 [..., d/group]   (the fp16 group minimum)
"""
from __future__ import annotations

import numpy as np

D_HEAD = 128
GROUP = 32
QMAX = 3  # 2**2 - 1 levels above the zero-point
BITS = (1, 2, 4)  # code widths of the codec


def levels(bits: int) -> int:
    """Levels above the zero-point of b-bit codes: 2**b - 1."""
    if bits not in BITS:
        raise ValueError(f"code width must be one of {BITS}")
    return (1 << bits) - 1


# --------------------------------------------------------------------------
# O1: rotation
# --------------------------------------------------------------------------
def hadamard_rotation(d: int = D_HEAD) -> np.ndarray:
    """Normalized Sylvester-order Hadamard matrix, fp64.

    H[i, j] = (-1)**popcount(i & j) / sqrt(d).  This is the matrix the
    in-place fast Walsh-Hadamard butterfly multiplies by (RotateKV abstract,
    item (i): the rotation keeps the efficiency of the FWHT).  Natural
    (Sylvester) order is a reading: the pages do not say which ordering.
    """
    if d <= 0 or d & (d - 1):
        raise ValueError("Hadamard size must be a power of two")
    idx = np.arange(d)
    bits = np.bitwise_and(idx[:, None], idx[None, :])
    parity = np.zeros_like(bits)
    while np.any(bits):
        parity ^= bits & 1
        bits = bits >> 1
    return np.where(parity == 1, -1.0, 1.0) / np.sqrt(float(d))


def permuted_hadamard_rotation(perm) -> np.ndarray:
    """Per-head rotation R_h = P_h . H for channel orders perm [H, d], fp64.

    Channel reordering ahead of the fast Walsh-Hadamard transform (RotateKV,
    IJCAI 2025 record, abstract item (i): the reordering adapts the rotation
    to where the outlier channels are while the transform stays the FWHT).
    The pages do not say how the order is applied; the reading here: the
    row is gathered first, (x P)_j = x[perm[j]], then rotated by H, so
    y = x P H and P[i, j] = 1 exactly when i == perm[j].
    """
    perm = np.asarray(perm)
    if perm.ndim != 2:
        raise ValueError("perm must be [heads, d]")
    n_heads, d = perm.shape
    H = hadamard_rotation(d)
    out = np.empty((n_heads, d, d))
    for h in range(n_heads):
        if sorted(perm[h].tolist()) != list(range(d)):
            raise ValueError("each row of perm must be a permutation of 0..d-1")
        P = np.zeros((d, d))
        P[perm[h], np.arange(d)] = 1.0
        out[h] = P @ H
    return out


def rotate_rows(x: np.ndarray, R: np.ndarray | None) -> np.ndarray:
    """y = x . R for row vectors x, in fp64, rounded once to fp32.

    Row-vector convention: a cache row k becomes k R, the query q becomes
    q R and the output o' becomes o' R^T (woor.ai page, "Key Details":
    applied before quantization, removed after attention).  R=None is the
    identity (inputs are only converted to fp32).
    """
    x64 = np.asarray(x, dtype=np.float64)
    if R is None:
        return x64.astype(np.float32)
    y64 = x64 @ np.asarray(R, dtype=np.float64)
    return y64.astype(np.float32)


# --------------------------------------------------------------------------
# O2-O4: group statistics, scale/zero, codes
# --------------------------------------------------------------------------
def quantize_rows(y32: np.ndarray, group: int = GROUP, bits: int = 2):
    """Asymmetric b-bit quantization of fp32 rows in channel groups
    (b = 2: INT2; L = 2**b - 1 levels above the zero-point).

    Per row and per group of `group` contiguous channels:
        mn, mx = min, max                       (exact)
        s32    = fp32( fp32(mx - mn) / L )      (IEEE fp32 ops)
        scale  = fp16_rne(s32);  zero = fp16_rne(mn + 0.0)
        if scale == 0: every code is 0
        else:  inv  = fp32(1 / fp32(scale))
               u    = fp32( fp32(y - fp32(zero)) * inv )
               code = clamp(rint_half_even(u), 0, L)
    Codes are taken against the stored fp16 scale and zero so that
    dequantization code*scale + zero is self-consistent.  Adding +0.0 to the
    minimum makes a zero minimum +0 whatever the signs of the group's zeros
    (the minimum of -0 and +0 is otherwise unspecified).

    Returns (codes uint8 [..., d], scales fp16 [..., d/group],
    zeros fp16 [..., d/group]).
    """
    y32 = np.asarray(y32)
    if y32.dtype != np.float32:
        raise TypeError("quantize_rows expects fp32 rows")
    d = y32.shape[-1]
    if d % group:
        raise ValueError("row length must be a multiple of the group size")
    ng = d // group
    qmax = levels(bits)
    yg = y32.reshape(*y32.shape[:-1], ng, group)
    mn = yg.min(axis=-1)
    mx = yg.max(axis=-1)
    rng32 = np.subtract(mx, mn, dtype=np.float32)
    s32 = np.divide(rng32, np.float32(qmax), dtype=np.float32)
    scale_h = s32.astype(np.float16)
    zero_h = np.add(mn, np.float32(0), dtype=np.float32).astype(np.float16)

    scale32 = scale_h.astype(np.float32)
    zero32 = zero_h.astype(np.float32)
    safe = np.where(scale32 == 0, np.float32(1), scale32)
    inv = np.divide(np.float32(1), safe, dtype=np.float32)
    diff = np.subtract(yg, zero32[..., None], dtype=np.float32)
    u = np.multiply(diff, inv[..., None], dtype=np.float32)
    code = np.clip(np.rint(u), 0, qmax)
    code = np.where((scale32 == 0)[..., None], 0, code)
    codes = code.astype(np.uint8).reshape(y32.shape)
    return codes, scale_h, zero_h


# --------------------------------------------------------------------------
# O5: packing
# --------------------------------------------------------------------------
def pack_codes(codes: np.ndarray, bits: int = 2) -> np.ndarray:
    """8/b codes of b bits per byte, first channel in the lowest bits.

    b = 2: byte j = c[4j] | c[4j+1] << 2 | c[4j+2] << 4 | c[4j+3] << 6
    b-bit: byte j = sum over i < 8/b of c[(8/b) j + i] << (b i)
    """
    qmax = levels(bits)
    per = 8 // bits
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % per:
        raise ValueError(f"row length must be a multiple of {per}")
    if np.any(codes > qmax):
        raise ValueError(f"codes must be in [0, {qmax}]")
    c = codes.reshape(*codes.shape[:-1], codes.shape[-1] // per, per).astype(np.uint32)
    packed = np.zeros(c.shape[:-1], np.uint32)
    for i in range(per):
        packed |= c[..., i] << (bits * i)
    return packed.astype(np.uint8)


def unpack_codes(packed: np.ndarray, bits: int = 2) -> np.ndarray:
    """Inverse of pack_codes: uint8 [..., d*b/8] -> uint8 codes [..., d]."""
    qmax = levels(bits)
    per = 8 // bits
    p = np.asarray(packed, dtype=np.uint8)
    parts = [(p >> (bits * i)) & qmax for i in range(per)]
    return np.stack(parts, axis=-1).reshape(*p.shape[:-1], p.shape[-1] * per)


# --------------------------------------------------------------------------
# O6: dequantization
# --------------------------------------------------------------------------
def dequantize(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
               group: int = GROUP) -> np.ndarray:
    """x_hat = code * scale + zero in fp64 (exact for fp16 scale/zero)."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    ng = d // group
    c = codes.reshape(*codes.shape[:-1], ng, group).astype(np.float64)
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)[..., None]
    z = np.asarray(zeros, dtype=np.float16).astype(np.float64)[..., None]
    return (c * s + z).reshape(codes.shape)


# --------------------------------------------------------------------------
# Write path: rotate -> quantize -> pack, for whole caches
# --------------------------------------------------------------------------
def quantize_cache(x: np.ndarray, R_heads=None, group: int = GROUP, bits: int = 2):
    """Quantize K or V given head-major rows x [B, H, T, d].

    R_heads: None (no rotation), a single [d, d] matrix used for every head,
    or [H, d, d] (one per head).  Returns (packed [B,H,T,d*bits/8] uint8,
    scales [B,H,T,d/group] fp16, zeros [B,H,T,d/group] fp16).
    """
    x = np.asarray(x)
    B, H, T, d = x.shape
    packed = np.empty((B, H, T, d * bits // 8), np.uint8)
    scales = np.empty((B, H, T, d // group), np.float16)
    zeros = np.empty((B, H, T, d // group), np.float16)
    for h in range(H):
        R = _head_matrix(R_heads, h)
        y = rotate_rows(x[:, h], R)
        codes, s, z = quantize_rows(y, group, bits)
        packed[:, h] = pack_codes(codes, bits)
        scales[:, h] = s
        zeros[:, h] = z
    return packed, scales, zeros


def _head_matrix(R_heads, h):
    if R_heads is None:
        return None
    R = np.asarray(R_heads)
    if R.ndim == 2:
        return R
    return R[h]


# --------------------------------------------------------------------------
# O7: decode attention over the INT2 cache (+ fp16 sink / residual tokens)
# --------------------------------------------------------------------------
def decode_attention(q, kcache, vcache, t_begin, t_end, R_heads=None,
                     group: int = GROUP, sink_k=None, sink_v=None,
                     res_k=None, res_v=None, softmax_scale=None):
    """One decode query per (batch, query head) against the cached tokens.

    q       [B, Hq, d]  (any float dtype; promoted to fp64)
    kcache  (codes [B,Hkv,T_cap,d*b/8], scales, zeros) in the rotated basis;
            the code width b (1, 2 or 4) follows from the codes' row length
    vcache  same for V (its width may differ from the keys')
    INT2 tokens are [t_begin, t_end).  sink_* / res_* are optional fp16
    [B, Hkv, n, d] tokens kept unquantized in the ORIGINAL basis.

    For query head h the KV head is h // (Hq // Hkv).  With R = R_{h_kv}:
        q'   = q R
        s_t  = softmax_scale * q' . k_hat_t        (INT2 tokens)
        s_t  = softmax_scale * q  . k_t            (fp16 tokens)
        p    = softmax over all tokens (max-subtracted, fp64)
        out  = (sum_INT2 p_t v_hat_t) R^T + sum_fp16 p_t v_t
    softmax_scale defaults to 1/sqrt(d).  The readout is the scaled
    dot-product attention of the woor.ai page ("What You Need to Know");
    the un-rotation is the removal "after the attention computation"
    (same page, "Key Details").  Returns fp64 [B, Hq, d].
    """
    q64 = np.asarray(q, dtype=np.float64)
    B, Hq, d = q64.shape
    kc, ks, kz = kcache
    vc, vs, vz = vcache
    Hkv = kc.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    kbits, vbits = 8 * kc.shape[-1] // d, 8 * vc.shape[-1] // d
    if softmax_scale is None or softmax_scale <= 0:
        softmax_scale = 1.0 / np.sqrt(float(d))
    n_int2 = t_end - t_begin
    out = np.zeros((B, Hq, d), np.float64)
    for b in range(B):
        for hk in range(Hkv):
            R = _head_matrix(R_heads, hk)
            R64 = None if R is None else np.asarray(R, dtype=np.float64)
            if n_int2 > 0:
                khat = dequantize(unpack_codes(kc[b, hk, t_begin:t_end], kbits),
                                  ks[b, hk, t_begin:t_end],
                                  kz[b, hk, t_begin:t_end], group)
                vhat = dequantize(unpack_codes(vc[b, hk, t_begin:t_end], vbits),
                                  vs[b, hk, t_begin:t_end],
                                  vz[b, hk, t_begin:t_end], group)
            else:
                khat = np.zeros((0, d))
                vhat = np.zeros((0, d))
            fk, fv = [], []
            for seg_k, seg_v in ((sink_k, sink_v), (res_k, res_v)):
                if seg_k is not None and np.asarray(seg_k).shape[2] > 0:
                    fk.append(np.asarray(seg_k[b, hk], dtype=np.float64))
                    fv.append(np.asarray(seg_v[b, hk], dtype=np.float64))
            fk = np.concatenate(fk, 0) if fk else np.zeros((0, d))
            fv = np.concatenate(fv, 0) if fv else np.zeros((0, d))
            if khat.shape[0] + fk.shape[0] == 0:
                raise ValueError("decode over zero tokens is undefined")
            for g in range(G):
                hq = hk * G + g
                qv = q64[b, hq]
                qr = qv if R64 is None else qv @ R64
                s_int2 = (khat @ qr) * softmax_scale
                s_f16 = (fk @ qv) * softmax_scale
                m = max(s_int2.max(initial=-np.inf), s_f16.max(initial=-np.inf))
                p_int2 = np.exp(s_int2 - m)
                p_f16 = np.exp(s_f16 - m)
                L = p_int2.sum() + p_f16.sum()
                o_rot = p_int2 @ vhat
                o = o_rot if R64 is None else o_rot @ R64.T
                o = o + p_f16 @ fv
                out[b, hq] = o / L
    return out


# --------------------------------------------------------------------------
# Pre-RoPE grouped-head rotation of the keys
# --------------------------------------------------------------------------
# RotateKV (IJCAI 2025 record, abstract item (ii)) rotates keys before the
# rotary position embedding is applied and across a group of heads, to keep
# RoPE from disturbing the outlier-aware rotation and to spread outliers
# over heads.  The record fixes neither RoPE nor the grouping; the readings
# used here:
#   * RoPE is the rotate-half form: channel i pairs with i + d/2, pair i
#     turns by the angle t * base**(-2i/d) at position t, base 10000;
#   * an INT2 key's position is its cache slot t; the decode query comes in
#     already position-embedded (post-RoPE), as a decode step produces it;
#   * the grouped-head rotation concatenates the pre-RoPE key rows of g
#     consecutive KV heads (head-major channels, head j of the group first
#     at channels j*d .. j*d + d - 1) and applies the normalized Sylvester
#     Hadamard matrix of size g*d; each head's d-channel slice of the result
#     is one cache row, quantized like any other;
#   * values carry no RoPE and keep the per-head Hadamard rotation;
#   * fp16 sink / residual keys are kept as a plain fp16 cache would keep
#     them: position-embedded, unrotated.
ROPE_BASE = 10000.0


def rope(x, positions, base: float = ROPE_BASE) -> np.ndarray:
    """Rotary position embedding of rows x [..., T, d] at positions [T], in
    fp64: for pair i (channels i and i + d/2) with angle a = t * base**(-2i/d),
    (x_i, x_{i+d/2}) -> (x_i cos a - x_{i+d/2} sin a, x_{i+d/2} cos a + x_i sin a)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    theta = base ** (-2.0 * np.arange(half) / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def grouped_hadamard_rotation(group_heads: int, d: int = D_HEAD) -> np.ndarray:
    """The rotation over the channels of a group of g heads: the normalized
    Sylvester Hadamard matrix of size g*d (fp64)."""
    return hadamard_rotation(group_heads * d)


def quantize_cache_grouped(x: np.ndarray, group_heads: int, group: int = GROUP, bits: int = 2):
    """Quantize pre-RoPE keys x [B, H, T, d] with the grouped-head rotation:
    the rows of heads g*k .. g*k + g - 1 are concatenated along channels,
    rotated by grouped_hadamard_rotation(g) (fp64, rounded once to fp32), and
    each head's d-channel slice is quantized and packed as a cache row.
    Returns (packed, scales, zeros) laid out as quantize_cache's."""
    x = np.asarray(x)
    B, H, T, d = x.shape
    g = group_heads
    if H % g:
        raise ValueError("the head count must be a multiple of the group size")
    Rg = grouped_hadamard_rotation(g, d)
    packed = np.empty((B, H, T, d * bits // 8), np.uint8)
    scales = np.empty((B, H, T, d // group), np.float16)
    zeros = np.empty((B, H, T, d // group), np.float16)
    for k in range(H // g):
        hs = range(g * k, g * k + g)
        cat = np.concatenate([x[:, h] for h in hs], axis=-1)          # [B, T, g*d]
        y = rotate_rows(cat, Rg)
        for j, h in enumerate(hs):
            codes, sc, z = quantize_rows(y[..., j * d:(j + 1) * d], group, bits)
            packed[:, h] = pack_codes(codes, bits)
            scales[:, h] = sc
            zeros[:, h] = z
    return packed, scales, zeros


def decode_attention_prerope(q, kcache, vcache, t_begin, t_end, group_heads,
                             rope_base: float = ROPE_BASE, group: int = GROUP,
                             sink_k=None, sink_v=None, res_k=None, res_v=None,
                             softmax_scale=None):
    """Decode attention over a cache whose keys hold the grouped-head
    rotation of pre-RoPE keys (quantize_cache_grouped) and whose values hold
    the per-head Hadamard rotation (quantize_cache with the Hadamard matrix).

    q [B, Hq, d] is post-RoPE.  For INT2 token t (cache slot t, position t)
    of KV head h in group k = h // g, slot j = h % g:
        k_t  = slice j of [k_hat_{g k, t}, ..., k_hat_{g k + g - 1, t}] R_g^T
        s_t  = softmax_scale * q . rope(k_t, t)
    fp16 sink / residual keys are post-RoPE already: s_t = softmax_scale q.k_t.
        out  = (sum_INT2 p_t v_hat_t) H^T + sum_fp16 p_t v_t
    Returns fp64 [B, Hq, d].
    """
    q64 = np.asarray(q, dtype=np.float64)
    B, Hq, d = q64.shape
    kc, ks, kz = kcache
    vc, vs, vz = vcache
    Hkv = kc.shape[1]
    g = group_heads
    if Hq % Hkv or Hkv % g:
        raise ValueError("Hq must be a multiple of Hkv, and Hkv of the group size")
    G = Hq // Hkv
    kbits, vbits = 8 * kc.shape[-1] // d, 8 * vc.shape[-1] // d
    if softmax_scale is None or softmax_scale <= 0:
        softmax_scale = 1.0 / np.sqrt(float(d))
    Rg = grouped_hadamard_rotation(g, d)
    Hv = hadamard_rotation(d)
    pos = np.arange(t_begin, t_end)
    out = np.zeros((B, Hq, d), np.float64)
    for b in range(B):
        kpre = np.zeros((Hkv, t_end - t_begin, d))
        if t_end > t_begin:
            for k in range(Hkv // g):
                hs = range(g * k, g * k + g)
                cat = np.concatenate([dequantize(unpack_codes(kc[b, h, t_begin:t_end], kbits),
                                                 ks[b, h, t_begin:t_end], kz[b, h, t_begin:t_end], group)
                                      for h in hs], axis=-1)
                un = cat @ Rg.T
                for j, h in enumerate(hs):
                    kpre[h] = un[:, j * d:(j + 1) * d]
        for hk in range(Hkv):
            khat = rope(kpre[hk], pos, rope_base)
            if t_end > t_begin:
                vhat = dequantize(unpack_codes(vc[b, hk, t_begin:t_end], vbits),
                                  vs[b, hk, t_begin:t_end], vz[b, hk, t_begin:t_end], group)
            else:
                vhat = np.zeros((0, d))
            fk, fv = [], []
            for seg_k, seg_v in ((sink_k, sink_v), (res_k, res_v)):
                if seg_k is not None and np.asarray(seg_k).shape[2] > 0:
                    fk.append(np.asarray(seg_k[b, hk], dtype=np.float64))
                    fv.append(np.asarray(seg_v[b, hk], dtype=np.float64))
            fk = np.concatenate(fk, 0) if fk else np.zeros((0, d))
            fv = np.concatenate(fv, 0) if fv else np.zeros((0, d))
            if khat.shape[0] + fk.shape[0] == 0:
                raise ValueError("decode over zero tokens is undefined")
            for gg in range(G):
                hq = hk * G + gg
                qv = q64[b, hq]
                s_int2 = (khat @ qv) * softmax_scale
                s_f16 = (fk @ qv) * softmax_scale
                m = max(s_int2.max(initial=-np.inf), s_f16.max(initial=-np.inf))
                p_int2 = np.exp(s_int2 - m)
                p_f16 = np.exp(s_f16 - m)
                L = p_int2.sum() + p_f16.sum()
                o = (p_int2 @ vhat) @ Hv.T + p_f16 @ fv
                out[b, hq] = o / L
    return out


# --------------------------------------------------------------------------
# Code-level tolerance helper for the rotated write path
# --------------------------------------------------------------------------
def tie_distance(x, R, scales, zeros, group: int = GROUP):
    """Distance of the exact fp64 quantizer argument to the nearest code
    boundary k + 1/2, per element: |u* - (floor(u*) + 1/2)| with
    u* = (x R - zero) / scale in fp64 using the given fp16 scale/zero.
    Elements whose group has scale 0 get +inf.  Used to decide whether a
    code disagreement sits at a rounding tie.
    """
    y64 = np.asarray(x, dtype=np.float64)
    if R is not None:
        y64 = y64 @ np.asarray(R, dtype=np.float64)
    d = y64.shape[-1]
    ng = d // group
    yg = y64.reshape(*y64.shape[:-1], ng, group)
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)[..., None]
    z = np.asarray(zeros, dtype=np.float16).astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (yg - z) / s
        dist = np.abs(u - (np.floor(u) + 0.5))
    dist = np.where(s == 0, np.inf, dist)
    return dist.reshape(y64.shape)
