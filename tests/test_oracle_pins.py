"""Pins for the CPU oracle: checks against things other than the oracle.

Each pin ties the oracle to something fixed outside it: a library routine
(scipy's Sylvester Hadamard, torch's scaled-dot-product attention), a
textbook matrix, hand-derived fixtures under tests/golden/, a closed-form
identity, or a brute-force loop on tiny inputs.  The mutation test at the
end plants plausible mistakes in a copy of the oracle (on the CPU) and
checks that some pin fails for every one of them.
"""
import inspect
import json
import math
import os
import types

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import kvq_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_orthogonal(rng, d):
    qm, rm = np.linalg.qr(rng.standard_normal((d, d)))
    return qm * np.sign(np.diag(rm))[None, :]


# ---------------------------------------------------------------- rotation
def pin_hadamard_scipy(orc):
    """Popcount definition == scipy's Sylvester construction (RotateKV (i))."""
    for d in (2, 4, 32, 128):
        H = orc.hadamard_rotation(d) * math.sqrt(d)
        assert np.array_equal(np.rint(H), scipy.linalg.hadamard(d))
        assert np.allclose(H, np.rint(H), atol=1e-12)


def pin_hadamard_golden4(orc):
    H4 = np.array(_load("hadamard4.json")["H4"], dtype=np.float64)
    assert np.allclose(orc.hadamard_rotation(4) * 2.0, H4, atol=1e-15)


def pin_hadamard_orthogonal(orc):
    H = orc.hadamard_rotation(128)
    Hi = np.rint(H * math.sqrt(128)).astype(np.int64)
    assert np.array_equal(Hi @ Hi.T, 128 * np.eye(128, dtype=np.int64))
    assert np.abs(H @ H.T - np.eye(128)).max() < 1e-14


def pin_perm_hadamard_gather(orc):
    """Channel reordering ahead of the transform (RotateKV (i)): x R_h equals
    gathering x in the head's channel order, then scipy's Sylvester Hadamard
    (normalized); one-hot rows give the Hadamard row of the inverse position;
    the identity order gives the plain Hadamard rotation."""
    rng = np.random.default_rng(17)
    d = 128
    perm = np.stack([rng.permutation(d) for _ in range(3)])
    R = orc.permuted_hadamard_rotation(perm)
    Hs = scipy.linalg.hadamard(d).astype(np.float64) / math.sqrt(d)
    x = rng.standard_normal((5, d))
    for h in range(3):
        assert np.allclose(x @ R[h], x[:, perm[h]] @ Hs, atol=1e-12)
        inv = np.argsort(perm[h])
        for k in (0, 1, 77):
            e = np.zeros(d)
            e[k] = 1.0
            assert np.allclose(e @ R[h], Hs[inv[k]], atol=1e-15)
        assert np.abs(R[h] @ R[h].T - np.eye(d)).max() < 1e-14
    ident = orc.permuted_hadamard_rotation(np.arange(d)[None])
    assert np.allclose(ident[0], orc.hadamard_rotation(d), atol=0)


def pin_rotate_onehot_dense(orc):
    """Row-vector convention: e_k R is row k of R (a non-symmetric R)."""
    rng = np.random.default_rng(7)
    R = _rand_orthogonal(rng, 128).astype(np.float32)
    for k in (0, 5, 127):
        e = np.zeros(128, np.float32)
        e[k] = 1
        y = orc.rotate_rows(e[None], R)[0]
        assert np.array_equal(y, R[k])


def pin_parseval_and_dot_invariance(orc):
    """|xR| = |x| and (qR).(kR) = q.k for orthogonal R (fp64 rotation)."""
    rng = np.random.default_rng(11)
    for R in (orc.hadamard_rotation(128), _rand_orthogonal(rng, 128)):
        x = rng.standard_normal((16, 128))
        y = orc.rotate_rows(x, R).astype(np.float64)
        rel = np.abs(np.linalg.norm(y, axis=1) / np.linalg.norm(x, axis=1) - 1)
        assert rel.max() < 1e-6          # fp32 rounding of the result only
        q = rng.standard_normal(128)
        qr = q @ R
        assert abs((qr @ (x @ R).T - q @ x.T)).max() < 1e-10


# --------------------------------------------------------------- quantizer
def _golden_group(case):
    vals = [np.float32(float(v)) for v in case["values"]]
    codes = list(case["codes"])
    if case.get("fill_pattern_repeat"):
        reps = 32 // len(vals)
        vals = vals * reps
        codes = codes * reps
    else:
        fill = np.float32(float(case["fill"]))
        codes = codes + [0] * (32 - len(vals))
        vals = vals + [fill] * (32 - len(vals))
    return np.array(vals, np.float32), np.array(codes, np.uint8)


def pin_quant_golden(orc):
    for case in _load("quant_group_cases.json")["cases"]:
        y, want_codes = _golden_group(case)
        if case.get("fill") is not None and not case.get("fill_pattern_repeat"):
            # the fill entries' codes follow from the fill value itself
            fill = np.float32(float(case["fill"]))
            want_codes = _fill_codes(case, want_codes, fill)
        row = np.tile(y, 4)[None]               # four identical groups
        codes, s, z = orc.quantize_rows(row)
        assert float(s[0, 0]) == float(case["scale"]), case["name"]
        assert float(z[0, 0]) == float(case["zero"]), case["name"]
        if "zero_bits" in case:
            assert int(z[0, 0].view(np.uint16)) == case["zero_bits"], case["name"]
        assert np.array_equal(codes[0, :32], want_codes), case["name"]


def _fill_codes(case, codes, fill):
    n = len(case["values"])
    vals = [np.float32(float(v)) for v in case["values"]]
    for i in range(n, 32):
        # the fill value equals one of the listed values; copy its code
        j = vals.index(fill)
        codes[i] = case["codes"][j]
    return codes


def pin_quant_grid_random(orc):
    """Grid data z + j*s (exact in fp32) is recovered exactly."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        z = np.float16(rng.uniform(-4, 4))
        s = np.float16(2.0 ** rng.uniform(-4, 1))
        j = rng.integers(0, 4, size=(4, 32))
        j[:, :4] = [0, 1, 2, 3]                   # every level present
        y64 = float(z) + j * float(s)
        y = y64.astype(np.float32)
        if not np.array_equal(y.astype(np.float64), y64):
            continue
        codes, sc, zz = orc.quantize_rows(y.reshape(1, 128))
        assert np.all(sc == s) and np.all(zz == z)
        assert np.array_equal(codes.reshape(4, 32), j.astype(np.uint8))
        xh = orc.dequantize(codes, sc, zz)
        assert np.array_equal(xh.reshape(4, 32), y64)


def pin_quant_nearest_level(orc):
    """Every code picks the nearest of the four levels of its group (fp32
    slop only), for random outlier data in both bases."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 128)) * np.where(np.arange(128) % 37 == 3, 20, 1)
    for R in (None, orc.hadamard_rotation(128)):
        y = orc.rotate_rows(x, R)
        codes, s, z = orc.quantize_rows(y)
        lv = (np.arange(4)[None, None, :] * s.astype(np.float64)[..., None]
              + z.astype(np.float64)[..., None])          # [64, 4, 4]
        yg = y.astype(np.float64).reshape(64, 4, 32)
        err = np.abs(yg[..., None] - lv[:, :, None, :])     # [64,4,32,4]
        chosen = np.take_along_axis(err, codes.reshape(64, 4, 32, 1).astype(np.int64), -1)[..., 0]
        best = err.min(-1)
        slop = 1e-6 * (np.abs(yg) + 1)
        assert np.all(chosen <= best + slop)


# ----------------------------------------------------------------- packing
def pin_pack_golden(orc):
    for case in _load("pack_row.json")["cases"]:
        c = np.array(case["codes"], np.uint8)[None]
        assert list(orc.pack_codes(c)[0]) == case["bytes"]
        assert np.array_equal(orc.unpack_codes(np.array([case["bytes"]], np.uint8)), c)


def pin_pack_roundtrip(orc):
    allb = np.arange(256, dtype=np.uint8)[None]
    assert np.array_equal(orc.pack_codes(orc.unpack_codes(allb)), allb)
    for b in range(256):
        c = orc.unpack_codes(np.array([[b]], np.uint8))[0]
        assert sum(int(c[i]) << (2 * i) for i in range(4)) == b


# ------------------------------------------------------- whole-cache write
def _grid_rows(rng, shape):
    """Grid data per group: z + j*s with j in 0..3 (levels 0 and 3 present
    in every group), z and s fp16 with |z| >= 0.25 and s in [1/4, 1], so the
    scale, zero and codes of such a row are z, s and j exactly, and a
    perturbation of a few fp32 ulps changes none of them."""
    *lead, d = shape
    ng = d // 32
    j = rng.integers(0, 4, size=(*lead, ng, 32))
    j[..., 0], j[..., 1] = 0, 3
    z = rng.choice([-1, 1], size=(*lead, ng)) * rng.uniform(0.25, 2.0, size=(*lead, ng))
    z = z.astype(np.float16)
    s = rng.uniform(0.25, 1.0, size=(*lead, ng)).astype(np.float16)
    y = z.astype(np.float64)[..., None] + j * s.astype(np.float64)[..., None]
    return y.reshape(*lead, d), j.reshape(*lead, d).astype(np.uint8), s, z


def _pack_by_hand(codes):
    """byte b = sum_i code[4b + i] << 2i, by explicit loops."""
    *lead, d = codes.shape
    flat = codes.reshape(-1, d)
    out = np.zeros((flat.shape[0], d // 4), np.uint8)
    for r in range(flat.shape[0]):
        for b in range(d // 4):
            out[r, b] = sum(int(flat[r, 4 * b + i]) << (2 * i) for i in range(4))
    return out.reshape(*lead, d // 4)


def pin_quantize_cache_per_head(orc):
    """Whole-cache write with a different rotation per head (OptR page, Key
    Details: one orthogonal rotation per head).  Rotated rows are chosen on
    a grid per head, the inputs are x = y R_h^T, and the expected codes,
    scales and zeros are the grid's own (codes packed by hand), for each of
    three non-symmetric per-head rotations: a dense QR rotation, a reordered
    Hadamard (permutation then scipy's Hadamard) and a signed permutation.
    Using one head's rotation for another, the transposed rotation, or the
    wrong head or batch slot gives different codes."""
    rng = np.random.default_rng(41)
    B, H, T, d = 2, 3, 5, 128
    Hs = scipy.linalg.hadamard(d).astype(np.float64) / math.sqrt(d)
    perm = rng.permutation(d)
    Pm = np.zeros((d, d))
    Pm[perm, np.arange(d)] = 1.0
    sp = rng.permutation(d)
    Sg = np.zeros((d, d))
    Sg[sp, np.arange(d)] = rng.choice([-1.0, 1.0], size=d)
    R = np.stack([_rand_orthogonal(rng, d), Pm @ Hs, Sg])
    for h in range(H):
        assert not np.allclose(R[h], R[h].T)
    y, j, s, z = _grid_rows(rng, (B, H, T, d))
    x = np.einsum("bhtc,hkc->bhtk", y, R).astype(np.float32)      # x = y R_h^T
    packed, sc, zz = orc.quantize_cache(x, R)
    assert packed.shape == (B, H, T, 32) and sc.shape == zz.shape == (B, H, T, 4)
    assert np.array_equal(sc, s) and np.array_equal(zz, z)
    assert np.array_equal(packed, _pack_by_hand(j))
    # one shared [d, d] matrix is used for every head
    y1, j1, s1, z1 = _grid_rows(rng, (1, H, 4, d))
    x1 = (y1 @ R[1].T).astype(np.float32)
    p1, sc1, zz1 = orc.quantize_cache(x1, R[1])
    assert np.array_equal(p1, _pack_by_hand(j1)) and np.array_equal(sc1, s1) and np.array_equal(zz1, z1)


def pin_tie_distance_dense(orc):
    """tie_distance takes the exact argument (x R - zero)/scale with the
    caller's R.  With a signed permutation R (non-symmetric) and rotated
    values y = x R chosen by hand on one group with scale 1 and zero 0:
    y = 0.5, 1.5, 2.5 sit at ties (distance 0), y = 0.75 and 2.25 at 0.25,
    y = 1 and 3 at 0.5; a scale-0 group gives +inf."""
    rng = np.random.default_rng(43)
    d = 128
    sp = rng.permutation(d)
    R = np.zeros((d, d))
    R[sp, np.arange(d)] = rng.choice([-1.0, 1.0], size=d)
    assert not np.allclose(R, R.T)
    y = np.zeros(d)
    vals = [0.5, 1.5, 2.5, 0.75, 2.25, 1.0, 3.0]
    want = [0.0, 0.0, 0.0, 0.25, 0.25, 0.5, 0.5]
    y[:len(vals)] = vals
    x = (y @ R.T)[None]                                  # exact: a signed permutation
    scales = np.array([[1.0, 1.0, 0.0, 1.0]], np.float16)
    zeros = np.zeros((1, 4), np.float16)
    dist = orc.tie_distance(x, R, scales, zeros)
    assert list(dist[0, :len(vals)]) == want
    assert np.all(np.isinf(dist[0, 64:96]))
    assert np.all(dist[0, 32:64] == 0.5)                 # y = 0 lies mid-way between ties


# ------------------------------------- pre-RoPE grouped-head rotation (keys)
def _rope_complex(x, t, base=10000.0):
    """Rotary embedding written with complex numbers: pair i of x (channels
    i and i + d/2) is the complex number x_i + 1j x_{i+d/2}, multiplied by
    exp(1j t theta_i), theta_i = exp(-ln(base) 2i/d)."""
    d = x.shape[-1]
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    theta = np.exp(-math.log(base) * 2.0 * np.arange(half) / d)
    w = z * np.exp(1j * t * theta)
    return np.concatenate([w.real, w.imag], axis=-1)


def pin_rope_golden_and_complex(orc):
    """Hand values for d = 4, base 10000 (theta = 1 and 0.01): e_0 at
    position 1 goes to (cos 1, 0, sin 1, 0); e_1 at position 2 to
    (0, cos 0.02, 0, sin 0.02); position 0 is the identity.  At d = 128 the
    rotate-half form equals the complex-number form."""
    r = orc.rope(np.array([[1.0, 0, 0, 0]]), [1])
    assert np.allclose(r, [[math.cos(1), 0, math.sin(1), 0]], atol=1e-15)
    r = orc.rope(np.array([[0.0, 1, 0, 0]]), [2])
    assert np.allclose(r, [[0, math.cos(0.02), 0, math.sin(0.02)]], atol=1e-15)
    rng = np.random.default_rng(51)
    x = rng.standard_normal((6, 128))
    assert np.array_equal(orc.rope(x, np.zeros(6)), x)
    pos = np.array([0, 1, 7, 100, 4095, 131071])
    want = np.stack([_rope_complex(x[i], pos[i]) for i in range(6)])
    assert np.allclose(orc.rope(x, pos), want, atol=1e-12)


def pin_rope_relative_position(orc):
    """rope(q, m) . rope(k, n) depends on m - n only, and rope keeps norms."""
    rng = np.random.default_rng(52)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, n in ((5, 3), (1000, 998), (70000, 3), (3, 70000)):
        a = orc.rope(q[None], [m])[0] @ orc.rope(k[None], [n])[0]
        b = orc.rope(q[None], [m - n])[0] @ k
        assert abs(a - b) < 1e-9 * (np.linalg.norm(q) * np.linalg.norm(k))
        assert abs(np.linalg.norm(orc.rope(k[None], [n])[0]) - np.linalg.norm(k)) < 1e-12


def pin_grouped_rotation(orc):
    """The rotation over g heads' channels is scipy's Hadamard of size 128 g
    (normalized), i.e. H_g kron H_128 with the head index as the high bits;
    g = 1 is the per-head Hadamard rotation."""
    for g in (1, 2, 4):
        Rg = orc.grouped_hadamard_rotation(g)
        n = 128 * g
        assert np.allclose(Rg, scipy.linalg.hadamard(n) / math.sqrt(n), atol=1e-15)
        assert np.allclose(Rg, np.kron(scipy.linalg.hadamard(g), scipy.linalg.hadamard(128)) / math.sqrt(n),
                           atol=1e-15)
        assert np.abs(Rg @ Rg.T - np.eye(n)).max() < 1e-13
    assert np.array_equal(orc.grouped_hadamard_rotation(1), orc.hadamard_rotation(128))


def pin_quantize_cache_grouped(orc):
    """Grouped write: rotated group rows chosen on a grid (per 32-channel
    group), inputs x = y R_g^T split into the g heads; the expected codes
    (packed by hand), scales and zeros are the grid's, for g = 2 and 4 with
    two head groups."""
    rng = np.random.default_rng(53)
    for g in (2, 4):
        B, H, T = 2, 2 * g, 3
        Rg = scipy.linalg.hadamard(128 * g) / math.sqrt(128 * g)
        y, j, s, z = _grid_rows(rng, (B, H // g, T, 128 * g))           # per head group
        xg = (y @ Rg.T).astype(np.float32)                               # [B, H/g, T, g*128]
        x = np.concatenate([xg[:, k, :, 128 * i:128 * (i + 1)][:, None]
                            for k in range(H // g) for i in range(g)], axis=1)
        packed, sc, zz = orc.quantize_cache_grouped(x, g)
        for k in range(H // g):
            for i in range(g):
                h = g * k + i
                sl = slice(128 * i, 128 * (i + 1))
                assert np.array_equal(packed[:, h], _pack_by_hand(j[:, k, :, sl]))
                assert np.array_equal(sc[:, h], s[:, k, :, 4 * i:4 * i + 4])
                assert np.array_equal(zz[:, h], z[:, k, :, 4 * i:4 * i + 4])


def _prerope_reference(q, kcache, vcache, t_begin, t_end, g, scale, sinks=None):
    """Plain loops: dequantized key rows of each head group concatenated,
    un-rotated with scipy's Hadamard (explicit sums), rotary-embedded with
    complex numbers at the cache slot, scores and softmax by loops, values
    un-rotated per head."""
    kp, ks, kz = kcache
    vp, vs, vz = vcache
    B, Hq, d = q.shape
    Hkv = kp.shape[1]
    G = Hq // Hkv
    n = 128 * g
    Hn = scipy.linalg.hadamard(n).astype(np.float64) / math.sqrt(n)
    H1 = scipy.linalg.hadamard(d).astype(np.float64) / math.sqrt(d)
    kc, vc = kvq_oracle.unpack_codes(kp), kvq_oracle.unpack_codes(vp)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        keys = {}
        for t in range(t_begin, t_end):
            for k in range(Hkv // g):
                cat = [int(kc[b, g * k + i, t, c]) * float(ks[b, g * k + i, t, c // 32])
                       + float(kz[b, g * k + i, t, c // 32]) for i in range(g) for c in range(d)]
                un = [sum(cat[m] * Hn[r, m] for m in range(n)) for r in range(n)]   # cat R^T
                for i in range(g):
                    keys[(g * k + i, t)] = _rope_complex(np.array(un[i * d:(i + 1) * d]), t)
        for hq in range(Hq):
            hk = hq // G
            sc, vals = [], []
            for t in range(t_begin, t_end):
                sc.append(scale * sum(float(q[b, hq, c]) * keys[(hk, t)][c] for c in range(d)))
                rot = [int(vc[b, hk, t, c]) * float(vs[b, hk, t, c // 32]) + float(vz[b, hk, t, c // 32])
                       for c in range(d)]
                vals.append([sum(rot[m] * H1[c, m] for m in range(d)) for c in range(d)])
            if sinks is not None:
                for kk, vv in zip(sinks[0][b, hk], sinks[1][b, hk]):
                    sc.append(scale * sum(float(q[b, hq, c]) * float(kk[c]) for c in range(d)))
                    vals.append([float(v) for v in vv])
            m = max(sc)
            p = [math.exp(x - m) for x in sc]
            L = sum(p)
            out[b, hq] = [sum(p[t] * vals[t][c] for t in range(len(p))) / L for c in range(d)]
    return out


def pin_decode_prerope_bruteforce(orc):
    """Decode over pre-RoPE grouped-rotated keys against plain loops, with
    two query heads per KV head, g = 2, INT2 slots [3, 7) and two fp16
    (post-RoPE) sink tokens."""
    rng = np.random.default_rng(54)
    B, Hkv, G, T, g = 1, 2, 2, 7, 2
    _, ks, kz, kp = _random_cache(rng, B, Hkv, T)
    _, vs, vz, vp = _random_cache(rng, B, Hkv, T)
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float16)
    sk = rng.standard_normal((B, Hkv, 2, 128)).astype(np.float16)
    sv = rng.standard_normal((B, Hkv, 2, 128)).astype(np.float16)
    out = orc.decode_attention_prerope(q, (kp, ks, kz), (vp, vs, vz), 3, T, g, sink_k=sk, sink_v=sv)
    ref = _prerope_reference(q.astype(np.float64), (kp, ks, kz), (vp, vs, vz), 3, T, g,
                             1 / math.sqrt(128), sinks=(sk, sv))
    assert np.abs(out - ref).max() <= 1e-11 * np.abs(ref).max()


def pin_decode_prerope_vs_sdpa(orc):
    """Against torch SDPA in fp64 on keys un-rotated (scipy's Hadamard of
    size 128 g) and rotary-embedded (complex form) at their slots, values
    un-rotated per head; g = 4, grouped-query heads, a softmax scale."""
    rng = np.random.default_rng(55)
    B, Hkv, G, T, g, tb = 2, 4, 2, 40, 4, 5
    kcodes, ks, kz, kp = _random_cache(rng, B, Hkv, T)
    vcodes, vs, vz, vp = _random_cache(rng, B, Hkv, T)
    q = rng.standard_normal((B, Hkv * G, 128))
    out = orc.decode_attention_prerope(q, (kp, ks, kz), (vp, vs, vz), tb, T, g, softmax_scale=0.05)
    n = 128 * g
    Hn = scipy.linalg.hadamard(n) / math.sqrt(n)
    H1 = scipy.linalg.hadamard(128) / math.sqrt(128)
    kr = _deq(kcodes, ks, kz)[:, :, tb:]                                  # [B, Hkv, T', 128]
    cat = kr.transpose(0, 2, 1, 3).reshape(B, T - tb, Hkv // g, n)       # head groups
    un = (cat @ Hn.T).reshape(B, T - tb, Hkv, 128).transpose(0, 2, 1, 3)
    pos = np.arange(tb, T)
    K = np.stack([np.stack([np.stack([_rope_complex(un[b, h, i], pos[i]) for i in range(T - tb)])
                            for h in range(Hkv)]) for b in range(B)])
    V = _deq(vcodes, vs, vz)[:, :, tb:] @ H1.T
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], torch.from_numpy(np.repeat(K, G, axis=1)),
        torch.from_numpy(np.repeat(V, G, axis=1)), scale=0.05)[:, :, 0].numpy()
    assert np.abs(out - ref).max() <= 1e-11 * np.abs(ref).max()


# ------------------------------------------------------ other code widths
def pin_quant_bits_grid(orc):
    """1- and 4-bit codes: grid data z + j*s, j in [0, 2**b - 1] with every
    level present, is recovered exactly (scale = s, zero = z, codes = j)."""
    rng = np.random.default_rng(13)
    for bits, L in ((1, 1), (4, 15)):
        done = 0
        for _ in range(400):
            z = np.float16(rng.uniform(-4, 4))
            s = np.float16(2.0 ** rng.uniform(-4, 0))
            j = rng.integers(0, L + 1, size=(4, 32))
            j[:, 0], j[:, 1] = 0, L
            y64 = float(z) + j * float(s)
            y = y64.astype(np.float32)
            if not np.array_equal(y.astype(np.float64), y64):
                continue
            codes, sc, zz = orc.quantize_rows(y.reshape(1, 128), bits=bits)
            assert np.all(sc == s) and np.all(zz == z), bits
            assert np.array_equal(codes.reshape(4, 32), j.astype(np.uint8)), bits
            assert np.array_equal(orc.dequantize(codes, sc, zz).reshape(4, 32), y64)
            done += 1
        assert done > 50


def pin_quant_bits_ramp(orc):
    """Hand-derived groups.  Ramp y_i = i, i = 0..31:
    4 bits: range 31, scale = fp16(31/15): 31/15 = 2.0666.., the fp16 step
    in [2, 4) is 2^-9, 2.0666../2^-9 = 1058.13, so scale = 1058 * 2^-9 =
    2.06640625; code_i = round(i / scale) in exact rationals (no i sits
    within 0.01 of a half).  1 bit: scale = 31, code = 1 exactly for
    i >= 16 (15/31 < 1/2 < 16/31)."""
    from fractions import Fraction
    y = np.tile(np.arange(32, dtype=np.float32), 4)[None]
    codes, s, z = orc.quantize_rows(y, bits=4)
    assert float(s[0, 0]) == 2.06640625 and float(z[0, 0]) == 0.0
    sc = Fraction(1058, 512)
    want = []
    for i in range(32):
        u = Fraction(i) / sc
        k = math.floor(u)
        assert abs(u - k - Fraction(1, 2)) > Fraction(1, 100)
        want.append(k + (1 if u - k > Fraction(1, 2) else 0))
    assert list(codes[0, :32]) == want
    assert want[-1] == 15 and want[1] == 0 and want[2] == 1
    codes1, s1, _ = orc.quantize_rows(y, bits=1)
    assert float(s1[0, 0]) == 31.0
    assert list(codes1[0, :32]) == [0] * 16 + [1] * 16


def pin_quant_bits_nearest(orc):
    """Every 1- and 4-bit code picks the nearest level of its group (fp32
    slop only), for random outlier data in both bases."""
    rng = np.random.default_rng(15)
    x = rng.standard_normal((32, 128)) * np.where(np.arange(128) % 29 == 5, 20, 1)
    for bits in (1, 4):
        L = (1 << bits) - 1
        for R in (None, orc.hadamard_rotation(128)):
            y = orc.rotate_rows(x, R)
            codes, s, z = orc.quantize_rows(y, bits=bits)
            lv = (np.arange(L + 1)[None, None, :] * s.astype(np.float64)[..., None]
                  + z.astype(np.float64)[..., None])
            yg = y.astype(np.float64).reshape(32, 4, 32)
            err = np.abs(yg[..., None] - lv[:, :, None, :])
            chosen = np.take_along_axis(err, codes.reshape(32, 4, 32, 1).astype(np.int64), -1)[..., 0]
            assert np.all(chosen <= err.min(-1) + 1e-6 * (np.abs(yg) + 1)), bits


def pin_pack_bits(orc):
    """Hand-packed bytes: 1 bit, codes 1,0,1,1,0,0,0,1 -> 1+4+8+128 = 141;
    4 bits, codes 3,12 -> 3 + 12*16 = 195, codes 15,0 -> 15.  Every byte
    value round-trips at each width."""
    c1 = np.array([[1, 0, 1, 1, 0, 0, 0, 1] * 2], np.uint8)
    assert list(orc.pack_codes(c1, bits=1)[0]) == [141, 141]
    c4 = np.array([[3, 12, 15, 0]], np.uint8)
    assert list(orc.pack_codes(c4, bits=4)[0]) == [195, 15]
    allb = np.arange(256, dtype=np.uint8)[None]
    for bits in (1, 4):
        c = orc.unpack_codes(allb, bits=bits)
        assert c.shape == (1, 256 * 8 // bits) and c.max() == (1 << bits) - 1
        assert np.array_equal(orc.pack_codes(c, bits=bits), allb)
    assert list(orc.unpack_codes(np.array([[141]], np.uint8), bits=1)[0]) == [1, 0, 1, 1, 0, 0, 0, 1]
    assert list(orc.unpack_codes(np.array([[195]], np.uint8), bits=4)[0]) == [3, 12]


def pin_decode_mixed_widths(orc):
    """Decode reads each cache at its own width: 2-bit caches re-encoded as
    4-bit codes (same levels, scales and zeros) give the same output; keys
    at 4 bits with values at 2 bits, and keys at 1 bit (codes 0/1 written at
    1 and at 2 bits) likewise."""
    rng = np.random.default_rng(17)
    B, H, T, d = 1, 2, 40, 128
    q = rng.standard_normal((B, 2 * H, d))
    kc, ks, kz, kp = _random_cache(rng, B, H, T)
    vc, vs, vz, vp = _random_cache(rng, B, H, T)
    ref = orc.decode_attention(q, (kp, ks, kz), (vp, vs, vz), 3, T)
    k4 = orc.pack_codes(orc.unpack_codes(kp), bits=4)
    v4 = orc.pack_codes(orc.unpack_codes(vp), bits=4)
    assert k4.shape[-1] == 64
    for kk, vv in (((k4, ks, kz), (vp, vs, vz)), ((k4, ks, kz), (v4, vs, vz)), ((kp, ks, kz), (v4, vs, vz))):
        assert np.allclose(orc.decode_attention(q, kk, vv, 3, T), ref, rtol=0, atol=1e-12)
    kb = orc.unpack_codes(kp) & 1                           # codes in {0, 1}
    r2 = orc.decode_attention(q, (orc.pack_codes(kb), ks, kz), (vp, vs, vz), 3, T)
    r1 = orc.decode_attention(q, (orc.pack_codes(kb, bits=1), ks, kz), (vp, vs, vz), 3, T)
    assert orc.pack_codes(kb, bits=1).shape[-1] == 16
    assert np.allclose(r1, r2, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ decode
def _random_cache(rng, B, H, T, d=128):
    codes = rng.integers(0, 4, size=(B, H, T, d)).astype(np.uint8)
    scales = rng.uniform(0.05, 0.6, size=(B, H, T, d // 32)).astype(np.float16)
    zeros = rng.uniform(-1.0, 0.2, size=(B, H, T, d // 32)).astype(np.float16)
    packed = kvq_oracle.pack_codes(codes)
    return codes, scales, zeros, packed


def _deq(codes, scales, zeros):
    c = codes.reshape(*codes.shape[:-1], 4, 32).astype(np.float64)
    return (c * scales.astype(np.float64)[..., None]
            + zeros.astype(np.float64)[..., None]).reshape(codes.shape)


def pin_decode_vs_sdpa(orc):
    """Rotate q / un-rotate o over an exact cache == plain attention in the
    original basis (torch SDPA, fp64), with GQA, dense per-head R and fp16
    sink / residual tokens."""
    rng = np.random.default_rng(9)
    B, Hkv, G, T, d = 2, 2, 2, 12, 128
    Hq = Hkv * G
    Rh = np.stack([_rand_orthogonal(rng, d) for _ in range(Hkv)])
    for R_heads, scale in ((Rh, None), (orc.hadamard_rotation(d), None), (None, 0.3)):
        kcodes, ks, kz, kp = _random_cache(rng, B, Hkv, T)
        vcodes, vs, vz, vp = _random_cache(rng, B, Hkv, T)
        sink_k = rng.standard_normal((B, Hkv, 2, d)).astype(np.float16)
        sink_v = rng.standard_normal((B, Hkv, 2, d)).astype(np.float16)
        res_k = rng.standard_normal((B, Hkv, 3, d)).astype(np.float16)
        res_v = rng.standard_normal((B, Hkv, 3, d)).astype(np.float16)
        q = rng.standard_normal((B, Hq, d))
        out = orc.decode_attention(q, (kp, ks, kz), (vp, vs, vz), 0, T, R_heads,
                                   sink_k=sink_k, sink_v=sink_v, res_k=res_k,
                                   res_v=res_v, softmax_scale=scale)
        kr = _deq(kcodes, ks, kz)
        vr = _deq(vcodes, vs, vz)
        if R_heads is not None:
            Rs = R_heads if R_heads.ndim == 3 else np.stack([R_heads] * Hkv)
            kr = np.einsum("bhtj,hcj->bhtc", kr, Rs)   # k = k_rot R^T
            vr = np.einsum("bhtj,hcj->bhtc", vr, Rs)
        K = np.concatenate([sink_k.astype(np.float64), kr, res_k.astype(np.float64)], 2)
        V = np.concatenate([sink_v.astype(np.float64), vr, res_v.astype(np.float64)], 2)
        Kq = torch.from_numpy(np.repeat(K, G, axis=1))
        Vq = torch.from_numpy(np.repeat(V, G, axis=1))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[:, :, None, :], Kq, Vq, scale=scale)[:, :, 0].numpy()
        assert np.abs(out - ref).max() <= 1e-11 * np.abs(ref).max()


def pin_decode_bruteforce(orc):
    """Plain loops over un-rotated tokens (k = k_hat R^T) with the original
    query, T <= 16, Hadamard built by scipy."""
    rng = np.random.default_rng(21)
    d, T = 128, 9
    R = scipy.linalg.hadamard(d) / math.sqrt(d)
    kcodes, ks, kz, kp = _random_cache(rng, 1, 1, T)
    vcodes, vs, vz, vp = _random_cache(rng, 1, 1, T)
    q = rng.standard_normal((1, 1, d)).astype(np.float16)
    out = orc.decode_attention(q, (kp, ks, kz), (vp, vs, vz), 0, T, R)[0, 0]

    qv = [float(v) for v in q[0, 0]]
    korig, vorig = [], []
    for t in range(T):
        for codes, sc, zz, dst in ((kcodes, ks, kz, korig), (vcodes, vs, vz, vorig)):
            rot = [int(codes[0, 0, t, c]) * float(sc[0, 0, t, c // 32])
                   + float(zz[0, 0, t, c // 32]) for c in range(d)]
            dst.append([sum(rot[j] * R[c, j] for j in range(d)) for c in range(d)])
    s = [sum(qv[c] * korig[t][c] for c in range(d)) / math.sqrt(d) for t in range(T)]
    m = max(s)
    p = [math.exp(x - m) for x in s]
    L = sum(p)
    ref = [sum(p[t] * vorig[t][c] for t in range(T)) / L for c in range(d)]
    assert np.abs(out - np.array(ref)).max() < 1e-12 * max(abs(r) for r in ref)


def pin_decode_large_scores(orc):
    """Scores of order 1e4 (x50 sink-like keys) stay finite: softmax is
    max-subtracted, and the result equals the limit (all mass on the top
    token)."""
    rng = np.random.default_rng(13)
    d, T = 128, 8
    kcodes, ks, kz, kp = _random_cache(rng, 1, 1, T)
    vcodes, vs, vz, vp = _random_cache(rng, 1, 1, T)
    sink_k = (rng.standard_normal((1, 1, 1, d)) * 50).astype(np.float16)
    sink_v = rng.standard_normal((1, 1, 1, d)).astype(np.float16)
    q = (sink_k[0, 0].astype(np.float64) * 2)          # aligned with the sink
    out = orc.decode_attention(q[None], (kp, ks, kz), (vp, vs, vz), 0, T, None,
                               sink_k=sink_k, sink_v=sink_v)
    assert np.all(np.isfinite(out))
    assert np.allclose(out[0, 0], sink_v[0, 0, 0].astype(np.float64), atol=1e-12)


PINS = [
    pin_hadamard_scipy, pin_hadamard_golden4, pin_hadamard_orthogonal,
    pin_perm_hadamard_gather, pin_rotate_onehot_dense, pin_parseval_and_dot_invariance,
    pin_quant_golden, pin_quant_grid_random, pin_quant_nearest_level,
    pin_pack_golden, pin_pack_roundtrip,
    pin_decode_vs_sdpa, pin_decode_bruteforce, pin_decode_large_scores,
    pin_quant_bits_grid, pin_quant_bits_ramp, pin_quant_bits_nearest, pin_pack_bits,
    pin_decode_mixed_widths, pin_quantize_cache_per_head, pin_tie_distance_dense,
    pin_rope_golden_and_complex, pin_rope_relative_position, pin_grouped_rotation,
    pin_quantize_cache_grouped, pin_decode_prerope_bruteforce, pin_decode_prerope_vs_sdpa,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(kvq_oracle)


# ---------------------------------------------------- properties and format
def test_hadamard_reduces_int2_error_on_outliers():
    """Hadamard rotation lowers INT2 error on outlier data (KVLinC abstract:
    the rotation reduces quantization error).  Property, not parity."""
    from workloads import config, kv_tokens
    cfg = config(1)
    H = kvq_oracle.hadamard_rotation(128)
    for which in ("K", "V"):
        x = kv_tokens(cfg, which).numpy()[0, :, 0]            # [T, d] fp32
        errs = []
        for R in (None, H):
            y = kvq_oracle.rotate_rows(x, R)
            c, s, z = kvq_oracle.quantize_rows(y)
            errs.append(np.mean((kvq_oracle.dequantize(c, s, z) - y) ** 2))
        assert errs[1] < 0.6 * errs[0]


def test_outlier_order_reduces_int2_error():
    """Reordering each head's channels by outlier magnitude ahead of the
    Hadamard transform lowers the INT2 reconstruction error further on
    outlier data (RotateKV abstract, item (i): the reordering adapts the
    rotation to the channel-wise outliers).  Property, not parity."""
    from workloads import config, small_config, kv_tokens, channel_orders
    cfg = small_config(config(2), B=1, T=256, Hkv=4, Hq=4)
    x = kv_tokens(cfg, "K").numpy()[0].transpose(1, 0, 2)          # [H, T, d]
    H = kvq_oracle.hadamard_rotation(128)
    Rp = kvq_oracle.permuted_hadamard_rotation(channel_orders(cfg))

    def mse(R, h):
        y = kvq_oracle.rotate_rows(x[h], R)
        c, s, z = kvq_oracle.quantize_rows(y)
        back = kvq_oracle.dequantize(c, s, z) @ np.asarray(R, np.float64).T
        return np.mean((back - x[h].astype(np.float64)) ** 2)

    plain = np.mean([mse(H, h) for h in range(cfg.Hkv)])
    ordered = np.mean([mse(Rp[h], h) for h in range(cfg.Hkv)])
    assert ordered < 0.9 * plain


def test_format_bits_per_element():
    """2-bit codes + fp16 scale and zero per 32 channels = 3 bits/element,
    18.75% of fp16 (the OptR page quotes roughly 75% savings, Key Details)."""
    x = np.random.default_rng(0).standard_normal((3, 128)).astype(np.float32)
    c, s, z = kvq_oracle.quantize_rows(x)
    p = kvq_oracle.pack_codes(c)
    nbytes = p.nbytes + s.nbytes + z.nbytes
    assert nbytes * 8 / x.size == 3.0
    assert nbytes / (x.size * 2) == 0.1875


def test_tie_distance_marks_half_integers():
    y = np.array([[0.0, 0.75, 0.125, 0.375] + [0.0] * 124], np.float32)
    c, s, z = kvq_oracle.quantize_rows(y)
    dist = kvq_oracle.tie_distance(y, None, s, z)
    assert dist[0, 2] == 0.0 and dist[0, 3] == 0.0
    assert dist[0, 1] == 0.5


# ----------------------------------------------------------- mutation test
MUTATIONS = [
    ("un-rotation with R instead of R^T", "o_rot @ R64.T", "o_rot @ R64"),
    ("query rotated by R^T", "qv @ R64\n", "qv @ R64.T\n"),
    ("zero-point dropped in dequantization", "(c * s + z)", "(c * s)"),
    ("round half up instead of half even", "np.clip(np.rint(u), 0, qmax)",
     "np.clip(np.floor(u + 0.5), 0, qmax)"),
    ("softmax scale 1/d", "1.0 / np.sqrt(float(d))", "1.0 / float(d)"),
    ("divisor 4 instead of 3", "np.float32(qmax), dtype", "np.float32(qmax + 1), dtype"),
    ("packing order swapped", "packed |= c[..., i] << (bits * i)",
     "packed |= c[..., per - 1 - i] << (bits * i)"),
    ("fp16 values taken from keys", "p_f16 @ fv", "p_f16 @ fk"),
    ("Hadamard parity or-ed", "parity ^= bits & 1", "parity |= bits & 1"),
    ("GQA head mapping interleaved", "hq = hk * G + g", "hq = g * Hkv + hk"),
    ("no max subtraction", "np.exp(s_int2 - m)", "np.exp(s_int2)"),
    ("zero from the max", "np.add(mn, np.float32(0)", "np.add(mx, np.float32(0)"),
    ("signed zero kept", "np.add(mn, np.float32(0), dtype=np.float32)", "mn"),
    ("no clamp", "np.clip(np.rint(u), 0, qmax)", "np.rint(u)"),
    ("rotation transposed", "x64 @ np.asarray(R, dtype=np.float64)",
     "x64 @ np.asarray(R, dtype=np.float64).T"),
    ("channel order applied inverted", "P[perm[h], np.arange(d)] = 1.0",
     "P[np.arange(d), perm[h]] = 1.0"),
    ("channel order after the transform", "out[h] = P @ H", "out[h] = H @ P"),
    ("2**b levels instead of 2**b - 1", "return (1 << bits) - 1", "return 1 << bits"),
    ("key width taken from the values", "kbits, vbits = 8 * kc.shape[-1] // d",
     "kbits, vbits = 8 * vc.shape[-1] // d"),
    ("unpack mask fixed at 2 bits", "& qmax for i in range(per)", "& 3 for i in range(per)"),
    ("1-bit divisor 2", "qmax = levels(bits)\n    yg", "qmax = max(levels(bits), 2)\n    yg"),
    ("head 0's rotation for every head", "R = _head_matrix(R_heads, h)\n        y = rotate_rows",
     "R = _head_matrix(R_heads, 0)\n        y = rotate_rows"),
    ("rows of the wrong head written", "y = rotate_rows(x[:, h], R)", "y = rotate_rows(x[:, H - 1 - h], R)"),
    ("tie distance with R^T", "y64 = y64 @ np.asarray(R, dtype=np.float64)",
     "y64 = y64 @ np.asarray(R, dtype=np.float64).T"),
    ("rotary sine sign flipped", "x2 * c + x1 * s", "x2 * c - x1 * s"),
    ("rotary pairs interleaved", "x1, x2 = x[..., :half], x[..., half:]",
     "x1, x2 = x[..., 0::2], x[..., 1::2]"),
    ("rotary frequencies base**(-i/d)", "base ** (-2.0 * np.arange(half) / d)",
     "base ** (-1.0 * np.arange(half) / d)"),
    ("key positions counted from the range start", "pos = np.arange(t_begin, t_end)",
     "pos = np.arange(0, t_end - t_begin)"),
    ("head order reversed in a group", "cat = np.concatenate([x[:, h] for h in hs], axis=-1)",
     "cat = np.concatenate([x[:, h] for h in reversed(hs)], axis=-1)"),
    ("grouped rotation over one head only", "return hadamard_rotation(group_heads * d)",
     "return np.kron(np.eye(group_heads), hadamard_rotation(d))"),
    ("values not un-rotated (pre-RoPE decode)", "o = (p_int2 @ vhat) @ Hv.T + p_f16 @ fv",
     "o = (p_int2 @ vhat) + p_f16 @ fv"),
]


def _mutant(old, new):
    src = inspect.getsource(kvq_oracle)
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    with np.errstate(all="ignore"):
        exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new):
    mod = _mutant(old, new)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:  # AssertionError, or the mutant crashing
            caught.append(pin.__name__)
    assert caught, f"no pin catches: {name}"
