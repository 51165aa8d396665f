"""GPU parity of the write kernels' quantizer where both sides see the same
rotated rows, and of the method's edge cases on every rotated writer.

The codes, scales and zeros of the format must be bit-exact given identical
rotated inputs (the quantizer of the format runs on rows already turned by
the head's rotation: "Output-Aware Rotation for INT2 KV-Cache
Quantization", woor.ai page, "Key Details").  A rotation computed
in fp32 on the GPU and in fp64 by the oracle rarely gives the same rounded
row, so these tests build inputs whose rotation is exact on both sides:

* Hadamard (plain and reordered): rows of the rotated basis are small
  integers z times fp32(1/sqrt(128)); the input x = z H / 128 is exact in
  fp16, the transform of x is exactly z in fp32 (multiples of 1/128 far below
  2^24), and z is restricted to values whose product with fp32(1/sqrt(128))
  rounds to the same fp32 as the oracle's fp64 rotation.  The test asserts
  that equality before comparing codes.  Scaling x by 2^-17 or 2^11 (exact)
  gives subnormal-scale and large-range groups.
* Dense: per-head signed permutation matrices, so x R is exact in both the
  matrix cores (the fp16 hi part is R itself, the lo part 0) and the oracle.

The rows cover constant groups (scale 0), zero rows, groups far from zero
relative to their spread (the clamped code form), two-level groups and
random rows, at 1, 2 and 4 bits, through the 4-heads-per-wave (Hkv = 4) and
one-head-per-wave (Hkv = 3) tilings.
"""
import json

import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O
import int2_rotated_kv_amd as kvq
from parity_util import (SENTINEL, require_gpu, empty_cache, cache_to_numpy, rot_matrix,
                         compare_codes_at_ties, normwise_rel_err)

pytestmark = pytest.mark.gpu
DEV = "cuda"
C32 = np.float32(1.0 / np.sqrt(128.0))
H_INT = np.rint(O.hadamard_rotation(128) * np.sqrt(128.0)).astype(np.int64)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _report(name, **kw):
    print(f"[exact] {name} " + json.dumps(kw), flush=True)


# nonzero integers whose scaled value rounds like the fp64 rotation
Z_OK = np.array([z for z in range(-15, 16)
                 if z != 0 and np.float32(np.float32(z) * C32) == np.float32(z / np.sqrt(128.0))])


def _z_rows(rng, n):
    """n rows of 128 integers in the rotated basis, by kind (row index mod 8):
    random; constant groups; zero row; groups far from zero (values 14/15 or
    -15/-14 in groups 0 and 2); two-level groups; random."""
    z = rng.choice(Z_OK, size=(n, 128))
    for r in range(n):
        kind = r % 8
        if kind == 1:
            for g in range(4):
                z[r, 32 * g:32 * g + 32] = rng.choice(Z_OK)
        elif kind == 2:
            z[r] = 0
        elif kind == 3:
            z[r, 0:32] = rng.choice([14, 15], size=32)
            z[r, 64:96] = rng.choice([-15, -14], size=32)
        elif kind == 4:
            for g in range(4):
                a, b = rng.choice(Z_OK, size=2, replace=False)
                z[r, 32 * g:32 * g + 32] = rng.choice([a, b], size=32)
    return z


def _exact_hadamard_inputs(rng, B, T, H, e, perm=None):
    """fp16 inputs [B, T, H, 128] whose rotation (Hadamard, or the reordered
    Hadamard with channel orders perm [H, 128]) is exactly fp32(z * c) * 2^e."""
    z = _z_rows(rng, B * T * H).reshape(B, T, H, 128)
    xq = (z @ H_INT).astype(np.float64) / 128.0 * 2.0 ** e       # the rotated-domain input x_pi
    x16 = xq.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), xq), "inputs not exact in fp16"
    if perm is not None:                                         # x[pi(j)] = x_pi[j]
        x = np.empty_like(x16)
        for h in range(H):
            x[:, :, h, perm[h]] = x16[:, :, h, :]
        x16 = x
    y = (z.astype(np.float32) * C32).astype(np.float32) * np.float32(2.0 ** e)
    return torch.from_numpy(x16), y


def _assert_bitexact(gpu, ora, what):
    gp, gs, gz = gpu
    op, os_, oz = ora
    n_code = int((O.unpack_codes(gp, 1 if gp.shape[-1] == 16 else 4 if gp.shape[-1] == 64 else 2)
                  != O.unpack_codes(op, 1 if op.shape[-1] == 16 else 4 if op.shape[-1] == 64 else 2)).sum())
    n_s = int((gs.view(np.uint16) != os_.view(np.uint16)).sum())
    n_z = int((gz.view(np.uint16) != oz.view(np.uint16)).sum())
    _report(what, code_mismatch=n_code, scale_mismatch=n_s, zero_mismatch=n_z, groups=int(gs.size))
    assert n_code == 0 and n_s == 0 and n_z == 0, what


@pytest.mark.parametrize("rot", ["hadamard", "perm"])
@pytest.mark.parametrize("Hkv", [4, 3])
@pytest.mark.parametrize("bits", [2, 1, 4])
def test_quantize_rotated_exact_bitexact(rot, Hkv, bits):
    """fp16 Hadamard / reordered-Hadamard writers: codes, scales and zeros
    bit-exact when the rotated rows are identical; three input scales
    (2^0, 2^-17: subnormal fp16 scales, 2^11: wide ranges), K and V sides
    in one call, slots at an offset with the others untouched."""
    rng = np.random.default_rng(100 + 10 * Hkv + bits)
    B, T, toff = 2, 45, 7
    perm = np.stack([rng.permutation(128) for _ in range(Hkv)]).astype(np.int32) if rot == "perm" else None
    Rm = rot_matrix(rot, perm)
    for e in (0, -17, 11):
        xk, yk = _exact_hadamard_inputs(rng, B, T, Hkv, e, perm)
        xv, yv = _exact_hadamard_inputs(rng, B, T, Hkv, e, perm)
        kc = empty_cache(B, Hkv, T + toff + 5, bits=bits)
        vc = empty_cache(B, Hkv, T + toff + 5, bits=bits)
        Rg = torch.as_tensor(perm, device=DEV) if rot == "perm" else None
        kvq.kvq_quantize(xk.to(DEV), xv.to(DEV), kc, vc, rot=rot, R=Rg, t_offset=toff)
        torch.cuda.synchronize()
        for x, y, c, side in ((xk, yk, kc, "K"), (xv, yv, vc, "V")):
            xh = x.permute(0, 2, 1, 3).contiguous().numpy()
            for h in range(Hkv):                              # the oracle sees the same rotated rows
                Rh = Rm[h] if rot == "perm" else Rm
                assert np.array_equal(O.rotate_rows(xh[:, h], Rh), y[:, :, h].astype(np.float32))
            ora = O.quantize_cache(xh, Rm, bits=bits)
            g = cache_to_numpy(c)
            _assert_bitexact(tuple(a[:, :, toff:toff + T] for a in g), ora,
                             f"{rot} Hkv={Hkv} bits={bits} 2^{e} {side}")
            for arr in (g[0], g[1].view(np.uint8), g[2].view(np.uint8)):
                assert np.all(arr[:, :, :toff] == SENTINEL) and np.all(arr[:, :, toff + T:] == SENTINEL)


def test_quantize_fp32_hadamard_exact_bitexact():
    """fp32 rows with the Hadamard rotation (the rows kernel): bit-exact on
    identical rotated rows, at the three input scales."""
    rng = np.random.default_rng(7)
    B, T, H = 2, 70, 3
    Rm = rot_matrix("hadamard")
    for e in (0, -17, 11):
        x16, y = _exact_hadamard_inputs(rng, B, T, H, e)
        x = x16.float()
        c = empty_cache(B, H, T)
        kvq.kvq_quantize(x.to(DEV), None, c, None, rot="hadamard")
        torch.cuda.synchronize()
        xh = x.permute(0, 2, 1, 3).contiguous().numpy()
        assert np.array_equal(O.rotate_rows(xh, Rm), y.transpose(0, 2, 1, 3))
        _assert_bitexact(cache_to_numpy(c), O.quantize_cache(xh, Rm), f"fp32 hadamard 2^{e}")


def _signed_permutations(rng, H):
    R = np.zeros((H, 128, 128), np.float32)
    for h in range(H):
        R[h, rng.permutation(128), np.arange(128)] = rng.choice([-1.0, 1.0], size=128)
    return R


def _special_rotated_rows(rng, n, wide):
    """Rows in the rotated basis (fp16 values) by kind: random normal;
    constant groups; zero rows; fp16 subnormals; values up to `wide` in
    magnitude; signed zeros among small values; groups far from zero."""
    y = rng.standard_normal((n, 128))
    for r in range(n):
        kind = r % 8
        if kind == 1:
            for g in range(4):
                y[r, 32 * g:32 * g + 32] = rng.standard_normal()
        elif kind == 2:
            y[r] = 0.0
        elif kind == 3:
            y[r] = rng.integers(-200, 200, size=128) * 2.0 ** -24
        elif kind == 4:
            y[r] = rng.uniform(-wide, wide, size=128)
        elif kind == 5:
            y[r] = np.where(rng.random(128) < 0.5, -0.0, 0.0)
            y[r, ::7] = rng.standard_normal(len(y[r, ::7])) * 1e-3
        elif kind == 6:
            y[r, 0:32] += 40.0
            y[r, 96:128] -= 25.0
    return y.astype(np.float16)


@pytest.mark.parametrize("bits", [2, 1, 4])
def test_quantize_dense_signed_permutation_bitexact(bits):
    """Dense writer with per-head signed permutations: x R is exact on both
    sides, so codes, scales and zeros are bit-exact, for constant, zero,
    subnormal, wide-range, signed-zero and offset groups; ragged T."""
    rng = np.random.default_rng(300 + bits)
    B, T, H = 2, 77, 4
    R = _signed_permutations(rng, H)
    # the widest rows keep (max - min) / L inside the fp16 range
    y = _special_rotated_rows(rng, B * T * H, 30000.0 if bits == 1 else 60000.0).reshape(B, T, H, 128)
    x = np.einsum("bthc,hkc->bthk", y.astype(np.float64), R.astype(np.float64)).astype(np.float16)
    xt = torch.from_numpy(x)
    kc = empty_cache(B, H, T, bits=bits)
    vc = empty_cache(B, H, T, bits=bits)
    Rg = torch.from_numpy(R).to(DEV)
    kvq.kvq_quantize(xt.to(DEV), xt.to(DEV), kc, vc, rot="dense", R=Rg)
    torch.cuda.synchronize()
    xh = xt.permute(0, 2, 1, 3).contiguous().numpy()
    for h in range(H):
        assert np.array_equal(O.rotate_rows(xh[:, h], R[h]), y[:, :, h].astype(np.float32))
    ora = O.quantize_cache(xh, R, bits=bits)
    for c, side in ((kc, "K"), (vc, "V")):
        _assert_bitexact(cache_to_numpy(c), ora, f"dense signed permutation bits={bits} {side}")


@pytest.mark.parametrize("rot,Hkv,bits", [("hadamard", 4, 2), ("hadamard", 3, 2), ("perm", 4, 2),
                                          ("dense", 4, 2), ("hadamard", 4, 4), ("hadamard", 3, 1),
                                          ("perm", 3, 4), ("dense", 3, 1), ("dense", 4, 4)])
def test_quantize_rotated_edge_rows_ties(rot, Hkv, bits):
    """Every rotated writer on edge rows with a general rotation (rounded
    transform on both sides), compared at rounding ties: zero rows,
    tiny-magnitude rows (subnormal fp16 scales), rows of standard deviation
    5000 in the rotated basis (wide ranges, with (max - min) / L inside the
    fp16 range at every width) and offset groups.  (Constant rotated groups
    need identical rotated rows, which the bit-exact tests above build: with
    a rounded transform their range is rounding noise.)"""
    rng = np.random.default_rng(500 + Hkv + bits)
    B, T = 2, 512            # enough elements that the 1e-5 mismatch bar allows a few ties
    perm = R = None
    if rot == "perm":
        perm = np.stack([rng.permutation(128) for _ in range(Hkv)]).astype(np.int32)
        Rm = O.permuted_hadamard_rotation(perm)
    elif rot == "dense":
        qm = [np.linalg.qr(rng.standard_normal((128, 128))) for _ in range(Hkv)]
        R = np.stack([q * np.sign(np.diag(r))[None, :] for q, r in qm]).astype(np.float32)
        Rm = R
    else:
        Rm = np.stack([rot_matrix("hadamard")] * Hkv)
    y = rng.standard_normal((B, T, Hkv, 128))
    kind = np.arange(T) % 4
    y[:, kind == 0] = 0.0
    y[:, kind == 1] *= 2.0 ** -19
    y[:, kind == 2] *= 5e3
    y[:, kind == 3, :, 0:32] += 9.0
    x = np.einsum("bthc,hkc->bthk", y, Rm.astype(np.float64)).astype(np.float16)
    xt = torch.from_numpy(x)
    c = empty_cache(B, Hkv, T, bits=bits)
    Rg = (torch.from_numpy(R).to(DEV) if rot == "dense" else
          torch.from_numpy(perm).to(DEV) if rot == "perm" else None)
    kvq.kvq_quantize(xt.to(DEV), None, c, None, rot=rot, R=Rg)
    torch.cuda.synchronize()
    gp, gs, gz = cache_to_numpy(c)
    xh = xt.permute(0, 2, 1, 3).contiguous().numpy()
    ora = O.quantize_cache(xh, Rm, bits=bits)
    assert np.all(gp[:, :, 0::4] == 0) and np.all(gs[:, :, 0::4] == 0) and np.all(gz[:, :, 0::4] == 0)
    tot = dict(elements=0, code_mismatch=0, group_scale_zero_diff=0)
    for h in range(Hkv):
        st = compare_codes_at_ties(xh[:, h], Rm[h], (gp[:, h], gs[:, h], gz[:, h]),
                                   tuple(a[:, h] for a in ora), max_frac=1.0, bits=bits)
        for k in tot:
            tot[k] += st[k]
    _report(f"edge rows {rot} Hkv={Hkv} bits={bits}", **tot)
    assert tot["code_mismatch"] <= 1e-5 * tot["elements"]
    sub = gs[:, :, 1::4].view(np.uint16)
    assert np.any((sub > 0) & (sub < 0x0400)), "no subnormal scale was produced"


# ------------------------------------------------------ decode, large scales
def _random_cache_np(rng, B, H, T, bits, big_frac):
    L = (1 << bits) - 1
    codes = rng.integers(0, L + 1, size=(B, H, T, 128)).astype(np.uint8)
    scales = rng.uniform(0.05, 0.5, size=(B, H, T, 4))
    zeros = rng.uniform(-1.0, 0.5, size=(B, H, T, 4))
    big = rng.random((B, H, T, 4)) < big_frac
    scales = np.where(big, rng.uniform(2e3, 6e4, size=scales.shape), scales)
    # zero-points near -L s / 2 centre the values, inside the fp16 range
    zeros = np.where(big, np.maximum(-0.5 * L * scales * rng.uniform(0.8, 1.2, size=scales.shape), -6e4), zeros)
    return O.pack_codes(codes, bits), scales.astype(np.float16), zeros.astype(np.float16)


@pytest.mark.parametrize("kind", ["g1_hadamard", "g1_none", "gqa_dense", "gqa_hadamard", "k4v2", "k1v1", "k4v4",
                                  "k4v4_gqa", "k2v1_gqa"])
def test_decode_large_value_scales(kind):
    """Value scales up to 6e4 (any finite fp16 scale is admitted): the G = 1
    kernel's fp16 weights p * s and the grouped-query kernel's fp16 value
    operands stay finite, and the output matches the oracle on the same
    cache bytes (fp32 query and output: the values themselves exceed fp16)."""
    rng = np.random.default_rng(sum(map(ord, kind)))
    B, Hkv, T = 2, 2, 900
    G = 4 if "gqa" in kind else 1
    Hq = Hkv * G
    kbits, vbits = {"k4v2": (4, 2), "k1v1": (1, 1), "k4v4": (4, 4), "k4v4_gqa": (4, 4),
                    "k2v1_gqa": (2, 1)}.get(kind, (2, 2))
    rot = "dense" if "dense" in kind else "none" if kind == "g1_none" else "hadamard"
    kp, ks, kz = _random_cache_np(rng, B, Hkv, T, kbits, 0.0)
    vp, vs, vz = _random_cache_np(rng, B, Hkv, T, vbits, 0.3)
    assert float(vs.max()) > 4e4
    R = None
    if rot == "dense":
        qm = [np.linalg.qr(rng.standard_normal((128, 128))) for _ in range(Hkv)]
        R = np.stack([q * np.sign(np.diag(r))[None, :] for q, r in qm]).astype(np.float32)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float32)
    kc = kvq.Int2Cache(*(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (kp, ks, kz)), bits=kbits)
    vc = kvq.Int2Cache(*(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (vp, vs, vz)), bits=vbits)
    out = kvq.kvq_decode_attention(torch.from_numpy(q).to(DEV), kc, vc, 3, T, rot=rot,
                                   R=torch.from_numpy(R).to(DEV) if R is not None else None)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o))
    Rm = R if rot == "dense" else rot_matrix(rot)
    ref = O.decode_attention(q, (kp, ks, kz), (vp, vs, vz), 3, T, Rm)
    err = normwise_rel_err(o, ref)
    _report(f"decode large value scales {kind}", err=err, max_abs_out=float(np.abs(ref).max()))
    assert err <= 2e-3



@pytest.mark.parametrize("kind", ["g1_hadamard", "g1_none", "gqa_dense", "k1v1", "k1v2", "k2v1", "k4v2", "k4v4",
                                  "k2v1_gqa"])
def test_decode_small_value_scales(kind):
    """Value scales in fp16's subnormal range (values of order 1e-6): every
    weight that enters an fp16 operand stays a normal fp16 number relative
    to its own head's values, so the output keeps the relative tolerance of
    ordinary inputs (fp32 query and output; the oracle on the same bytes)."""
    rng = np.random.default_rng(7 + sum(map(ord, kind)))
    B, Hkv, T = 2, 2, 900
    G = 4 if "gqa" in kind else 1
    Hq = Hkv * G
    kbits, vbits = {"k1v1": (1, 1), "k1v2": (1, 2), "k2v1": (2, 1), "k4v2": (4, 2), "k4v4": (4, 4),
                    "k2v1_gqa": (2, 1)}.get(kind, (2, 2))
    rot = "dense" if "dense" in kind else "none" if kind == "g1_none" else "hadamard"
    kp, ks, kz = _random_cache_np(rng, B, Hkv, T, kbits, 0.0)
    L = (1 << vbits) - 1
    vp = O.pack_codes(rng.integers(0, L + 1, size=(B, Hkv, T, 128)).astype(np.uint8), vbits)
    vs = rng.uniform(1e-7, 3e-6, size=(B, Hkv, T, 4))
    vz = -0.5 * L * vs * rng.uniform(0.8, 1.2, size=vs.shape)
    vs, vz = vs.astype(np.float16), vz.astype(np.float16)
    assert float(vs.max()) < 2.0 ** -14                # every value scale is an fp16 subnormal
    R = None
    if rot == "dense":
        qm = [np.linalg.qr(rng.standard_normal((128, 128))) for _ in range(Hkv)]
        R = np.stack([q * np.sign(np.diag(r))[None, :] for q, r in qm]).astype(np.float32)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float32)
    kc = kvq.Int2Cache(*(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (kp, ks, kz)), bits=kbits)
    vc = kvq.Int2Cache(*(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (vp, vs, vz)), bits=vbits)
    out = kvq.kvq_decode_attention(torch.from_numpy(q).to(DEV), kc, vc, 3, T, rot=rot,
                                   R=torch.from_numpy(R).to(DEV) if R is not None else None)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    Rm = R if rot == "dense" else rot_matrix(rot)
    ref = O.decode_attention(q, (kp, ks, kz), (vp, vs, vz), 3, T, Rm)
    err = normwise_rel_err(o, ref)
    _report(f"decode small value scales {kind}", err=err, max_abs_out=float(np.abs(ref).max()))
    assert err <= 2e-3