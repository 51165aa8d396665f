"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bars:
* quantize with no rotation: codes, scales and zeros bit-exact;
* quantize with a rotation: <= 1e-5 of codes differ, each by one and at a
  rounding tie (or in a group whose scale/zero is one fp16 ulp off);
* decode: normwise relative error <= 2e-3 per (batch, query head) row
  against the oracle run on the same cache bytes.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O
import workloads as W
import int2_rotated_kv_amd as kvq
from parity_util import (SENTINEL, require_gpu, empty_cache, cache_to_numpy,
                         cache_from_numpy, rot_matrix, compare_codes_at_ties,
                         normwise_rel_err, elementwise_rel_err)

pytestmark = pytest.mark.gpu
DEV = "cuda"
ATTN_TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _report(name, **kw):
    print(f"[parity] {name} " + json.dumps(kw), flush=True)


def _rot_arg(rot, R):
    """The R argument of the library for a rotation: fp32 matrices (dense),
    int32 channel orders (perm) or None."""
    if rot == "dense":
        return torch.as_tensor(R, dtype=torch.float32, device=DEV).contiguous()
    if rot == "perm":
        return torch.as_tensor(R, dtype=torch.int32, device=DEV).contiguous()
    return None


# ------------------------------------------------------------ quantize
def _gpu_quantize(x_tok, rot, R=None, T_cap=None, t_offset=0, side="K"):
    B, T, H, d = x_tok.shape
    T_cap = T_cap or (T + t_offset)
    c = empty_cache(B, H, T_cap)
    xg = x_tok.to(DEV)
    Rg = _rot_arg(rot, R)
    if side == "K":
        kvq.kvq_quantize(xg, None, c, None, rot=rot, R=Rg, t_offset=t_offset)
    else:
        kvq.kvq_quantize(None, xg, None, c, rot=rot, R=Rg, t_offset=t_offset)
    torch.cuda.synchronize()
    return cache_to_numpy(c)


def _oracle_quantize(x_tok, rot, R=None, bits=2):
    x = x_tok.permute(0, 2, 1, 3).contiguous().numpy()   # [B, H, T, d]
    return O.quantize_cache(x, rot_matrix(rot, R), bits=bits)


def _outlier_rows(rng, shape, dtype):
    x = rng.standard_normal(shape)
    x[..., 3] *= 20
    x[..., 77] *= 12
    return torch.from_numpy(x.astype(dtype))


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_quantize_no_rotation_bitexact(dtype):
    """Ragged T (not a multiple of the 64-token block), t_offset > 0, three
    heads, two batches; regions outside the written slots stay untouched."""
    rng = np.random.default_rng(1)
    x = _outlier_rows(rng, (2, 203, 3, 128), dtype)
    toff, T_cap = 5, 230
    gp, gs, gz = _gpu_quantize(x, "none", T_cap=T_cap, t_offset=toff)
    op, os_, oz = _oracle_quantize(x, "none")
    sl = slice(toff, toff + 203)
    assert np.array_equal(gp[:, :, sl], op)
    assert np.array_equal(gs[:, :, sl].view(np.uint16), os_.view(np.uint16))
    assert np.array_equal(gz[:, :, sl].view(np.uint16), oz.view(np.uint16))
    for arr in (gp, gs.view(np.uint8), gz.view(np.uint8)):
        assert np.all(arr[:, :, :toff] == SENTINEL)
        assert np.all(arr[:, :, toff + 203:] == SENTINEL)


def _golden_rows():
    import test_oracle_pins as P
    rows = []
    for case in P._load("quant_group_cases.json")["cases"]:
        y, _ = P._golden_group(case)
        rows.append(np.tile(y, 4))
    return np.stack(rows).astype(np.float32)


def test_quantize_special_groups_bitexact():
    """Hand-derived golden groups (ties, constant group, clamps, subnormal
    scale), fp16 subnormals, signed zeros and wide-range groups, fp32 input."""
    rng = np.random.default_rng(2)
    rows = [_golden_rows()]
    sub = (rng.integers(-60, 60, size=(8, 128)) * 2.0 ** -24).astype(np.float32)
    rows.append(sub)                                   # fp16-subnormal values
    z = np.zeros((4, 128), np.float32)
    z[1] = -0.0
    z[2, ::2] = -0.0
    z[3, 5] = 1e-30
    rows.append(z)
    wide = rng.uniform(-60000, 60000, size=(8, 128)).astype(np.float32)
    rows.append(wide)
    grid = []
    for _ in range(8):
        zz = np.float16(rng.uniform(-8, 8))
        ss = np.float16(2.0 ** rng.uniform(-6, 2))
        j = rng.integers(0, 4, size=128)
        grid.append((float(zz) + j * float(ss)))
    rows.append(np.array(grid, np.float32))
    y = np.concatenate(rows)
    x = torch.from_numpy(y.reshape(1, -1, 1, 128))
    gp, gs, gz = _gpu_quantize(x, "none")
    op, os_, oz = _oracle_quantize(x, "none")
    assert np.array_equal(gp, op)
    assert np.array_equal(gs.view(np.uint16), os_.view(np.uint16))
    assert np.array_equal(gz.view(np.uint16), oz.view(np.uint16))


def test_quantize_strided_input_and_value_side():
    """Non-contiguous input (padded rows, device-side view) through the V
    side of the call."""
    rng = np.random.default_rng(3)
    big = _outlier_rows(rng, (2, 70, 2, 256), np.float16).to(DEV)
    x = big[..., 64:192]                                # channel stride 1, padded rows
    assert not x.is_contiguous() and x.stride(3) == 1
    c = empty_cache(2, 2, 70)
    kvq.kvq_quantize(None, x, None, c, rot="none")
    torch.cuda.synchronize()
    gp, gs, gz = cache_to_numpy(c)
    op, os_, oz = _oracle_quantize(x.cpu().contiguous(), "none")
    assert np.array_equal(gp, op)
    assert np.array_equal(gs.view(np.uint16), os_.view(np.uint16))
    assert np.array_equal(gz.view(np.uint16), oz.view(np.uint16))


@pytest.mark.parametrize("cid", [1, 2])
def test_quantize_hadamard_ties(cid):
    """Configs 1 (fp32, T=1024) and 2 (fp16, 32 heads, T=4096)."""
    cfg = W.config(cid)
    for which in ("K", "V"):
        x = W.kv_tokens(cfg, which)
        gpu = _gpu_quantize(x, "hadamard")
        ora = _oracle_quantize(x, "hadamard")
        xr = x.permute(0, 2, 1, 3).contiguous().numpy()
        st = compare_codes_at_ties(xr, rot_matrix("hadamard"), gpu, ora)
        _report(f"quantize_hadamard c{cid} {which}", **st)


@pytest.mark.parametrize("T,toff", [(300, 0), (517, 9), (1, 0), (33, 40)])
def test_quantize_dense_rotation_ties(T, toff):
    """Dense per-head rotation (MFMA path): ragged token counts (not a
    multiple of the 512-token block), t_offset, three heads, two batches."""
    cfg = W.small_config(W.config(4), B=2, T=T, Hkv=3, Hq=3, t_new=0)
    R = W.dense_rotations(cfg)
    for which in ("K", "V"):
        x = W.kv_tokens(cfg, which)
        gp, gs, gz = _gpu_quantize(x, "dense", R=R, T_cap=T + toff + 7, t_offset=toff)
        sl = slice(toff, toff + T)
        gpu = (gp[:, :, sl], gs[:, :, sl], gz[:, :, sl])
        for arr in (gp, gs.view(np.uint8), gz.view(np.uint8)):
            assert np.all(arr[:, :, :toff] == SENTINEL)
            assert np.all(arr[:, :, toff + T:] == SENTINEL)
        ora = _oracle_quantize(x, "dense", R)
        xr = x.permute(0, 2, 1, 3).contiguous().numpy()
        # per-head rotation: compare head by head
        for h in range(cfg.Hkv):
            st = compare_codes_at_ties(xr[:, h], R[h], tuple(a[:, h] for a in gpu),
                                       tuple(a[:, h] for a in ora))
        _report(f"quantize_dense T={T} {which}", **st)


@pytest.mark.parametrize("T,toff", [(100, 5), (64, 0), (1, 63)])
def test_quantize_hadamard_fp16_ragged_offset(T, toff):
    """The fp16 Hadamard kernel on a ragged token count (a partial 64-token
    tile) written at a token offset into a larger cache; slots outside the
    range keep their sentinel bytes."""
    cfg = W.small_config(W.config(2), B=2, T=T, Hkv=3, Hq=3)
    for which in ("K", "V"):
        x = W.kv_tokens(cfg, which)
        gp, gs, gz = _gpu_quantize(x, "hadamard", T_cap=T + toff + 5, t_offset=toff, side=which)
        sl = slice(toff, toff + T)
        for arr in (gp, gs.view(np.uint8), gz.view(np.uint8)):
            assert np.all(arr[:, :, :toff] == SENTINEL)
            assert np.all(arr[:, :, toff + T:] == SENTINEL)
        gpu = (gp[:, :, sl], gs[:, :, sl], gz[:, :, sl])
        ora = _oracle_quantize(x, "hadamard")
        xr = x.permute(0, 2, 1, 3).contiguous().numpy()
        st = compare_codes_at_ties(xr, rot_matrix("hadamard"), gpu, ora)
        _report(f"quantize_hadamard ragged T={T} toff={toff} {which}", **st)


@pytest.mark.parametrize("rot", ["hadamard", "dense"])
def test_quantize_offset_groups(rot):
    """Rows whose rotated groups sit far from zero relative to their spread
    (zero about 12 scales away in half of the groups), so waves take both
    forms of the rotated quantizer (the one that folds 1/scale into the
    first FMA is only used while every group has |zero| <= 8 scale)."""
    rng = np.random.default_rng(11)
    B, T, H, d = 2, 1030, 2, 128      # enough elements for the 1e-5 mismatch bar to allow a few ties
    y = 0.3 * rng.standard_normal((B, T, H, d))
    off = np.zeros(d)
    off[0:32] = 6.0
    off[64:96] = -6.0
    y[:, 1::2] += off                                  # odd tokens: offset groups 0 and 2
    if rot == "hadamard":
        R = None
        Rh = [rot_matrix("hadamard")] * H              # symmetric and orthogonal: its own inverse
    else:
        R = W.dense_rotations(W.small_config(W.config(4), B=B, T=T, Hkv=H, Hq=H, t_new=0))
        Rh = [R[h].astype(np.float64) for h in range(H)]
    # rows x with x R = y (R orthogonal: x = y R^T)
    x = np.stack([y[:, :, h] @ Rh[h].T for h in range(H)], axis=2)
    x = torch.from_numpy(x.astype(np.float16))
    gpu = _gpu_quantize(x, rot, R=R)
    ora = _oracle_quantize(x, rot, R)
    xr = x.permute(0, 2, 1, 3).contiguous().numpy()
    zs = ora[2].astype(np.float64) / np.maximum(ora[1].astype(np.float64), 1e-30)
    assert (np.abs(zs) > 8).any() and (np.abs(zs) <= 8).any()
    tot = dict(elements=0, code_mismatch=0, group_scale_zero_diff=0)
    for h in range(H):
        st = compare_codes_at_ties(xr[:, h], Rh[h] if rot == "dense" else rot_matrix("hadamard"),
                                   tuple(a[:, h] for a in gpu), tuple(a[:, h] for a in ora), max_frac=1.0)
        _report(f"quantize offset groups {rot} h={h}", **st)
        for k in tot:
            tot[k] += st[k]
    assert tot["code_mismatch"] <= 1e-5 * tot["elements"]


@pytest.mark.parametrize("order", ["outliers", "random"])
def test_quantize_perm_hadamard_ties(order):
    """Channel reordering ahead of the Hadamard transform (per-head orders:
    sorted by outlier magnitude, or random), ragged token count, offset."""
    cfg = W.small_config(W.config(2), B=2, T=1000, Hkv=3, Hq=3)
    if order == "outliers":
        perm = W.channel_orders(cfg)
    else:
        rng = np.random.default_rng(5)
        perm = np.stack([rng.permutation(128) for _ in range(cfg.Hkv)]).astype(np.int32)
    Rh = O.permuted_hadamard_rotation(perm)
    tot = dict(elements=0, code_mismatch=0, group_scale_zero_diff=0)
    for which in ("K", "V"):
        x = W.kv_tokens(cfg, which)
        gp, gs, gz = _gpu_quantize(x, "perm", R=perm, T_cap=cfg.T + 9, t_offset=9, side=which)
        gpu = (gp[:, :, 9:], gs[:, :, 9:], gz[:, :, 9:])
        ora = _oracle_quantize(x, "perm", perm)
        xr = x.permute(0, 2, 1, 3).contiguous().numpy()
        for h in range(cfg.Hkv):
            # per head: every mismatch at a tie; the fraction is checked over the whole call
            st = compare_codes_at_ties(xr[:, h], Rh[h], tuple(a[:, h] for a in gpu),
                                       tuple(a[:, h] for a in ora), max_frac=1.0)
            for k in tot:
                tot[k] += st[k]
    assert tot["code_mismatch"] <= 1e-5 * tot["elements"]
    _report(f"quantize_perm {order}", **tot)


def test_quantize_dense_config4_slice():
    """Config 4 shapes on the prefill slice (32768 new tokens of one
    sequence, all 8 heads)."""
    cfg = W.config(4)
    R = W.dense_rotations(cfg)
    t0, t1 = cfg.quant_range
    x = W.kv_tokens(cfg, "K", b0=0, b1=1, t0=t0, t1=t1)
    gpu = _gpu_quantize(x, "dense", R=R)
    ora = _oracle_quantize(x, "dense", R)
    xr = x.permute(0, 2, 1, 3).contiguous().numpy()
    tot = dict(elements=0, code_mismatch=0, group_scale_zero_diff=0)
    for h in range(cfg.Hkv):
        st = compare_codes_at_ties(xr[:, h], R[h], tuple(a[:, h] for a in gpu),
                                   tuple(a[:, h] for a in ora))
        for k in tot:
            tot[k] += st[k]
    assert tot["code_mismatch"] <= 1e-5 * tot["elements"]
    _report("quantize_dense c4 slice", **tot)


def test_quantize_both_sides_one_call():
    cfg = W.small_config(W.config(2), T=300, Hkv=4, Hq=4)
    K = W.kv_tokens(cfg, "K").to(DEV)
    V = W.kv_tokens(cfg, "V").to(DEV)
    ck, cv = empty_cache(1, 4, 300), empty_cache(1, 4, 300)
    kvq.kvq_quantize(K, V, ck, cv, rot="hadamard")
    torch.cuda.synchronize()
    for x, c in ((K, ck), (V, cv)):
        ora = _oracle_quantize(x.cpu(), "hadamard")
        xr = x.cpu().permute(0, 2, 1, 3).contiguous().numpy()
        compare_codes_at_ties(xr, rot_matrix("hadamard"), cache_to_numpy(c), ora)


# -------------------------------------------------------------- decode
def _decode_case(cfg, rot="hadamard", R=None, t_begin=None, t_end=None, n_sink=None,
                 n_res=None, scale=0.0, seed_q=None, name=""):
    """Oracle-quantized cache uploaded to the GPU; GPU decode vs oracle decode."""
    tb0, te0 = cfg.int2_range
    t_begin = tb0 if t_begin is None else t_begin
    t_end = te0 if t_end is None else t_end
    n_sink = cfg.n_sink if n_sink is None else n_sink
    n_res = cfg.n_res if n_res is None else n_res
    K = W.kv_tokens(cfg, "K")
    V = W.kv_tokens(cfg, "V")
    Rm = rot_matrix(rot, R)
    kh = K.permute(0, 2, 1, 3).contiguous().numpy()
    vh = V.permute(0, 2, 1, 3).contiguous().numpy()
    kcache = O.quantize_cache(kh, Rm)
    vcache = O.quantize_cache(vh, Rm)
    q = W.queries(cfg)
    sink = lambda a: np.ascontiguousarray(a[:, :, :n_sink]).astype(np.float16)
    resw = lambda a: np.ascontiguousarray(a[:, :, cfg.T - n_res:]).astype(np.float16)
    sk, sv = (sink(kh), sink(vh)) if n_sink else (None, None)
    rk, rv = (resw(kh), resw(vh)) if n_res else (None, None)
    ref = O.decode_attention(q.numpy(), kcache, vcache, t_begin, t_end, Rm,
                             sink_k=sk, sink_v=sv, res_k=rk, res_v=rv,
                             softmax_scale=scale if scale > 0 else None)
    up = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    Rg = _rot_arg(rot, R)
    out = kvq.kvq_decode_attention(q.to(DEV), cache_from_numpy(*kcache),
                                   cache_from_numpy(*vcache), t_begin, t_end, rot=rot,
                                   R=Rg, sink_k=up(sk), sink_v=up(sv), res_k=up(rk),
                                   res_v=up(rv), softmax_scale=scale)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    err = normwise_rel_err(out, ref)
    _report(f"decode {name or cfg.name}", normwise=err, elementwise=elementwise_rel_err(out, ref))
    assert np.all(np.isfinite(out))
    assert err <= ATTN_TOL
    return out, ref


def test_decode_config1_fp32():
    _decode_case(W.config(1), name="c1")


def test_decode_config2():
    _decode_case(W.config(2), name="c2")


@pytest.mark.parametrize("T", [1, 31, 33, 97, 300])
def test_decode_ragged_lengths(T):
    cfg = W.small_config(W.config(2), T=T, Hkv=3, Hq=3, B=2)
    _decode_case(cfg, name=f"ragged T={T}")


def test_decode_token_subrange_and_scale():
    cfg = W.small_config(W.config(3), T=500, Hkv=4, Hq=4, B=2)
    _decode_case(cfg, t_begin=37, t_end=411, scale=0.05, name="subrange")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_gqa_dense_rotation(G):
    cfg = W.small_config(W.config(4), T=700, B=2, Hkv=2, Hq=2 * G, t_new=0)
    R = W.dense_rotations(cfg)
    _decode_case(cfg, rot="dense", R=R, name=f"dense G={G}")


def test_decode_gqa_hadamard_g3():
    cfg = W.small_config(W.config(2), T=257, B=1, Hkv=2, Hq=6)
    _decode_case(cfg, name="G=3")


def test_decode_no_rotation():
    cfg = W.small_config(W.config(2), T=129, B=1, Hkv=2, Hq=2)
    _decode_case(cfg, rot="none", name="rot none")


def test_decode_sinks_and_residual():
    cfg = W.small_config(W.config(5), T=900, B=2, Hkv=3, Hq=3)
    _decode_case(cfg, name="sinks+res full")
    _decode_case(cfg, n_sink=0, n_res=0, name="sinks+res INT2 only")


def test_decode_fp16_tokens_only():
    cfg = W.small_config(W.config(5), T=200, B=1, Hkv=2, Hq=4)
    _decode_case(cfg, t_begin=4, t_end=4, n_sink=4, n_res=60, name="fp16 only")


def test_decode_fp16_tokens_dense_gqa():
    """Sinks and a ragged residual segment (73 fp16 tokens: more than one
    batch of rows in flight) with a dense rotation and four query heads per
    KV head."""
    cfg = W.small_config(W.config(4), T=700, B=2, Hkv=2, Hq=8, t_new=0)
    R = W.dense_rotations(cfg)
    _decode_case(cfg, rot="dense", R=R, t_begin=3, t_end=630, n_sink=3, n_res=70,
                 name="dense G=4 sinks+res")
    _decode_case(cfg, rot="dense", R=R, t_begin=0, t_end=700, n_sink=0, n_res=1,
                 name="dense G=4 one residual token")


@pytest.mark.parametrize("Hq,t_begin,t_end", [(2, 9, 60), (2, 5, 1000), (8, 7, 40), (8, 5, 1000),
                                             (8, 16, 1000), (2, 13, 77)])
def test_decode_shifted_tile_grid(Hq, t_begin, t_end):
    """A cache whose T_cap is a multiple of 16 with an INT2 range starting
    off a 16-row boundary: the tile grid starts t_begin mod 16 rows early and
    the first tile is masked below t_begin (for one and four query heads per
    KV head, a range inside a single tile masked at both ends, and ranges over
    many tiles)."""
    cfg = W.small_config(W.config(4), T=1024, B=2, Hkv=2, Hq=Hq, t_new=0)
    R = W.dense_rotations(cfg)
    _decode_case(cfg, rot="dense", R=R, t_begin=t_begin, t_end=t_end, n_sink=0, n_res=0,
                 name=f"shifted grid Hq={Hq} [{t_begin},{t_end})")
    cfg2 = W.small_config(W.config(2), T=1024, B=1, Hkv=2, Hq=Hq)
    _decode_case(cfg2, t_begin=t_begin, t_end=t_end, n_sink=0, n_res=0,
                 name=f"shifted grid hadamard Hq={Hq} [{t_begin},{t_end})")


@pytest.mark.parametrize("Hq", [3, 12])
def test_decode_perm_hadamard(Hq):
    """Reordered Hadamard rotation on the read path: q gathered in the
    head's order before the transform, the output scattered back after it;
    with sinks and residual tokens (original basis) and an INT2 range off a
    16-row boundary; one and four query heads per KV head."""
    cfg = W.small_config(W.config(5), T=1024, B=2, Hkv=3, Hq=Hq)
    rng = np.random.default_rng(23)
    perm = np.stack([rng.permutation(128) for _ in range(cfg.Hkv)]).astype(np.int32)
    _decode_case(cfg, rot="perm", R=perm, name=f"perm Hq={Hq}")
    _decode_case(cfg, rot="perm", R=perm, n_sink=0, n_res=0, name=f"perm Hq={Hq} INT2 only")


def test_decode_max_fp16_tokens():
    """The largest fp16 segment the library accepts (8192 sink + residual
    tokens) next to a short INT2 range."""
    cfg = W.small_config(W.config(5), T=8400, B=1, Hkv=2, Hq=2)
    _decode_case(cfg, t_begin=4, t_end=208, n_sink=4, n_res=8188, name="8192 fp16 tokens")


@pytest.mark.parametrize("Hq", [1, 2])
def test_decode_many_splits(Hq):
    """One KV head over a long range: about 500 splits per head, so
    the merge runs over many partials (one and two query heads)."""
    cfg = W.small_config(W.config(3), T=131072 + 37, B=1, Hkv=1, Hq=Hq)
    _decode_case(cfg, name=f"many splits Hq={Hq}")


@pytest.mark.parametrize("G", [2, 8])
def test_decode_gqa_hadamard(G):
    cfg = W.small_config(W.config(2), T=777, B=2, Hkv=2, Hq=2 * G)
    _decode_case(cfg, name=f"hadamard G={G}")


def test_decode_gqa_fp32_query():
    """fp32 queries (and fp32 output) with four query heads per KV head."""
    cfg = W.small_config(W.config(1), T=500, B=2, Hkv=2, Hq=8)
    _decode_case(cfg, name="fp32 q G=4")


@pytest.mark.parametrize("cid,Hkv,Hq,rot", [(5, 3, 3, "hadamard"), (4, 2, 8, "dense"), (2, 2, 2, "perm")])
def test_decode_varlen(cid, Hkv, Hq, rot):
    """Variable-length batch (kvq_decode_attention_varlen): sequence b
    attends to INT2 tokens [t_begin, t_ends[b]) of its own cache rows, plus
    the batch's fp16 tokens when the workload has them.  Ends include an
    empty range, a single token, ranges inside one tile and a full range."""
    T = 1024
    extra = dict(t_new=0) if cid == 4 else {}
    cfg = W.small_config(W.config(cid), T=T, B=5, Hkv=Hkv, Hq=Hq, **extra)
    tb = cfg.n_sink if cfg.n_sink else 3
    te_max = T - cfg.n_res
    ends = np.array([tb, tb + 1, tb + 40, tb + 333, te_max], np.int32)
    R = W.dense_rotations(cfg) if rot == "dense" else (
        np.stack([np.random.default_rng(9).permutation(128) for _ in range(cfg.Hkv)]).astype(np.int32)
        if rot == "perm" else None)
    Rm = rot_matrix(rot, R)
    K = W.kv_tokens(cfg, "K")
    V = W.kv_tokens(cfg, "V")
    kh = K.permute(0, 2, 1, 3).contiguous().numpy()
    vh = V.permute(0, 2, 1, 3).contiguous().numpy()
    kcache = O.quantize_cache(kh, Rm)
    vcache = O.quantize_cache(vh, Rm)
    q = W.queries(cfg)
    fp16 = {}
    if cfg.n_sink or cfg.n_res:
        fp16 = dict(sink_k=np.ascontiguousarray(kh[:, :, :cfg.n_sink]).astype(np.float16),
                    sink_v=np.ascontiguousarray(vh[:, :, :cfg.n_sink]).astype(np.float16),
                    res_k=np.ascontiguousarray(kh[:, :, T - cfg.n_res:]).astype(np.float16),
                    res_v=np.ascontiguousarray(vh[:, :, T - cfg.n_res:]).astype(np.float16))
    up = {k: torch.from_numpy(v).to(DEV) for k, v in fp16.items()}
    out = kvq.kvq_decode_attention(q.to(DEV), cache_from_numpy(*kcache), cache_from_numpy(*vcache),
                                   tb, te_max, rot=rot, R=_rot_arg(rot, R),
                                   t_ends=torch.from_numpy(ends).to(DEV), **up)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    for b in range(cfg.B):
        sl = lambda c: tuple(a[b:b + 1] for a in c)
        kwb = {k: v[b:b + 1] for k, v in fp16.items()}
        if ends[b] == tb and not fp16:
            assert np.all(out[b] == 0.0)                   # no token at all: zero output
            continue
        ref = O.decode_attention(q.numpy()[b:b + 1], sl(kcache), sl(vcache), tb, int(ends[b]), Rm, **kwb)
        err = normwise_rel_err(out[b:b + 1], ref)
        _report(f"decode varlen {rot} c{cid} b={b} [{tb},{ends[b]})", normwise=err)
        assert err <= ATTN_TOL


# ------------------------------------------------------------- paged caches
def _page_layout(rng, B, T_cap, P, spare=3):
    """A block table [B, T_cap/P] over a shuffled pool of pages (plus a few
    unused ones), and the pool size."""
    per = T_cap // P
    n_pages = B * per + spare
    pool = rng.permutation(n_pages)[:B * per]
    return pool.reshape(B, per).astype(np.int32), n_pages


def _to_pages(cache, table, n_pages, P):
    """Contiguous (codes, scales, zeros) [B, H, T, ...] -> paged arrays
    [n_pages, H, P, ...] (unused pages hold the sentinel)."""
    out = []
    for arr in cache:
        B, H, T = arr.shape[:3]
        pg = np.zeros((n_pages, H, P) + arr.shape[3:], arr.dtype)
        for b in range(B):
            for j in range(T // P):
                pg[table[b, j]] = arr[b, :, j * P:(j + 1) * P]
        out.append(pg)
    return out


@pytest.mark.parametrize("cid,Hkv,Hq,rot,P,tb", [(2, 2, 2, "hadamard", 128, 5), (4, 2, 8, "dense", 64, 0),
                                                 (5, 2, 2, "hadamard", 192, 4), (2, 3, 3, "perm", 64, 70)])
def test_decode_paged(cid, Hkv, Hq, rot, P, tb):
    """Paged decode (block table over a shuffled page pool, per-sequence
    ends): each sequence against the oracle on the same rows, and against
    the contiguous variable-length call over the same bytes."""
    T = 768
    extra = dict(t_new=0) if cid == 4 else {}
    cfg = W.small_config(W.config(cid), T=T, B=3, Hkv=Hkv, Hq=Hq, **extra)
    rng = np.random.default_rng(100 + cid)
    R = W.dense_rotations(cfg) if rot == "dense" else (W.channel_orders(cfg) if rot == "perm" else None)
    Rm = rot_matrix(rot, R)
    K = W.kv_tokens(cfg, "K")
    V = W.kv_tokens(cfg, "V")
    kh = K.permute(0, 2, 1, 3).contiguous().numpy()
    vh = V.permute(0, 2, 1, 3).contiguous().numpy()
    kcache = O.quantize_cache(kh, Rm)
    vcache = O.quantize_cache(vh, Rm)
    table, n_pages = _page_layout(rng, cfg.B, T, P)
    te_max = T - cfg.n_res
    tb = cfg.n_sink if cfg.n_sink else tb
    ends = np.array([te_max, tb + 1 + int(rng.integers(0, te_max - tb - 1)), tb + 64 + 3], np.int32)
    fp16 = {}
    if cfg.n_sink or cfg.n_res:
        fp16 = dict(sink_k=np.ascontiguousarray(kh[:, :, :cfg.n_sink]).astype(np.float16),
                    sink_v=np.ascontiguousarray(vh[:, :, :cfg.n_sink]).astype(np.float16),
                    res_k=np.ascontiguousarray(kh[:, :, T - cfg.n_res:]).astype(np.float16),
                    res_v=np.ascontiguousarray(vh[:, :, T - cfg.n_res:]).astype(np.float16))
    up = {k: torch.from_numpy(v).to(DEV) for k, v in fp16.items()}
    kp = kvq.PagedCache(*[torch.from_numpy(a).to(DEV) for a in _to_pages(kcache, table, n_pages, P)])
    vp = kvq.PagedCache(*[torch.from_numpy(a).to(DEV) for a in _to_pages(vcache, table, n_pages, P)])
    q = W.queries(cfg)
    tends = torch.from_numpy(ends).to(DEV)
    out = kvq.kvq_decode_attention_paged(q.to(DEV), kp, vp, tb, tends, te_max,
                                         torch.from_numpy(table).to(DEV), rot=rot, R=_rot_arg(rot, R), **up)
    flat = kvq.kvq_decode_attention(q.to(DEV), cache_from_numpy(*kcache), cache_from_numpy(*vcache),
                                    tb, te_max, rot=rot, R=_rot_arg(rot, R), t_ends=tends, **up)
    torch.cuda.synchronize()
    out, flat = out.float().cpu().numpy(), flat.float().cpu().numpy()
    worst = 0.0
    for b in range(cfg.B):
        sl = lambda c: tuple(a[b:b + 1] for a in c)
        kwb = {k: v[b:b + 1] for k, v in fp16.items()}
        ref = O.decode_attention(q.numpy()[b:b + 1], sl(kcache), sl(vcache), tb, int(ends[b]), Rm, **kwb)
        worst = max(worst, normwise_rel_err(out[b:b + 1], ref))
    err_flat = normwise_rel_err(out, flat)
    _report(f"decode paged {rot} c{cid} P={P} tb={tb}", normwise=worst, vs_contiguous=err_flat)
    assert worst <= ATTN_TOL and err_flat <= 1e-3


@pytest.mark.parametrize("rot,Hkv,P,f32", [("hadamard", 4, 128, False), ("perm", 3, 64, False),
                                           ("none", 2, 64, False), ("dense", 4, 128, False),
                                           ("hadamard", 3, 64, True)])
def test_quantize_paged(rot, Hkv, P, f32):
    """Paged decode-step appends and prefills: sequence b's rows at its own
    offset through the block table; pages not addressed keep their sentinel
    bytes, a table entry outside the pool drops its rows, and the written
    rows gathered back match the contiguous per-sequence write.  Every
    write kernel: fp16 (reordered) Hadamard, no rotation, dense R, fp32 rows."""
    cfg = W.small_config(W.config(2), B=3, T=150, Hkv=Hkv, Hq=Hkv)
    perm = (W.channel_orders(cfg) if rot == "perm" else
            W.dense_rotations(cfg) if rot == "dense" else None)
    rng = np.random.default_rng(7)
    T_cap = 4 * P
    table, n_pages = _page_layout(rng, cfg.B, T_cap, P)
    table[2, 1] = n_pages + 5                       # out of the pool: those rows are dropped
    offs = np.array([0, 37, P - 20], np.int32)      # the last crosses into page 1
    K = W.kv_tokens(cfg, "K")
    if f32:
        K = K.float()
    kp = kvq.PagedCache.empty(n_pages, Hkv, P)
    for t in (kp.codes, kp.scales.view(torch.uint8), kp.zeros.view(torch.uint8)):
        t.fill_(SENTINEL)
    Rg = _rot_arg(rot, perm)
    kvq.kvq_quantize_paged(K.to(DEV), None, kp, None, torch.from_numpy(offs).to(DEV),
                           torch.from_numpy(table).to(DEV), rot=rot, R=Rg)
    flat = empty_cache(cfg.B, Hkv, T_cap)
    kvq.kvq_quantize(K.to(DEV), None, flat, None, rot=rot, R=Rg, t_offsets=torch.from_numpy(offs).to(DEV))
    torch.cuda.synchronize()
    pc = cache_to_numpy(kp)
    fc = cache_to_numpy(flat)
    written = np.zeros((n_pages, P), bool)
    for b in range(cfg.B):
        for t in range(cfg.T):
            slot = int(offs[b]) + t
            page = int(table[b, slot // P])
            if page >= n_pages:
                continue
            written[page, slot % P] = True
            for a_p, a_f in zip(pc, fc):
                assert np.array_equal(a_p[page, :, slot % P].view(np.uint8), a_f[b, :, slot].view(np.uint8))
    for a_p in pc:                                   # nothing else was touched
        assert np.all(np.moveaxis(a_p.view(np.uint8), 1, 2)[~written] == SENTINEL)
    _report(f"quantize paged {rot}{' fp32' if f32 else ''} P={P}", rows=int(written.sum()))
    assert written.sum() < cfg.B * cfg.T             # the dropped page's rows are missing


# ------------------------------------------------ other code widths (1, 4 bits)
@pytest.mark.parametrize("kbits,vbits,rot", [(4, 2, "hadamard"), (1, 4, "hadamard"), (4, 4, "perm"),
                                             (1, 1, "perm"), (4, 2, "dense"), (1, 4, "dense"),
                                             (4, 4, "dense")])
def test_quantize_bits_ties(kbits, vbits, rot):
    """b-bit write path (keys and values at their own widths): codes, fp16
    scales and zeros against the oracle's b-bit codec, compared at rounding
    ties as for 2 bits; a ragged token count at an offset, so the first 9
    slots and the rows past T_new keep their sentinel bytes."""
    cfg = W.small_config(W.config(2), B=2, T=700, Hkv=3, Hq=3)
    perm = (W.channel_orders(cfg) if rot == "perm" else
            W.dense_rotations(cfg) if rot == "dense" else None)
    Rm = rot_matrix(rot, perm)
    K = W.kv_tokens(cfg, "K")
    V = W.kv_tokens(cfg, "V")
    T_cap = cfg.T + 20
    kc = empty_cache(cfg.B, cfg.Hkv, T_cap, bits=kbits)
    vc = empty_cache(cfg.B, cfg.Hkv, T_cap, bits=vbits)
    kvq.kvq_quantize(K.to(DEV), V.to(DEV), kc, vc, rot=rot, R=_rot_arg(rot, perm), t_offset=9)
    torch.cuda.synchronize()
    tot = dict(elements=0, code_mismatch=0, group_scale_zero_diff=0)
    for x, c, bits in ((K, kc, kbits), (V, vc, vbits)):
        gp, gs, gz = cache_to_numpy(c)
        assert gp.shape[-1] == 16 * bits
        for arr in (gp, gs.view(np.uint8), gz.view(np.uint8)):       # untouched slots
            assert np.all(arr[:, :, :9] == SENTINEL) and np.all(arr[:, :, 9 + cfg.T:] == SENTINEL)
        xh = x.permute(0, 2, 1, 3).contiguous().numpy()
        ora = O.quantize_cache(xh, Rm, bits=bits)
        for h in range(cfg.Hkv):
            Rh = Rm[h] if rot in ("perm", "dense") else Rm
            st = compare_codes_at_ties(xh[:, h], Rh, tuple(a[:, h, 9:9 + cfg.T] for a in (gp, gs, gz)),
                                       tuple(a[:, h] for a in ora), max_frac=1.0, bits=bits)
            for k in tot:
                tot[k] += st[k]
    _report(f"quantize bits K{kbits}V{vbits} {rot}", **tot)
    assert tot["code_mismatch"] <= 1e-5 * tot["elements"]


@pytest.mark.parametrize("kbits,vbits,rot,cid,G", [
    (4, 2, "hadamard", 2, 1), (2, 4, "hadamard", 2, 1), (1, 1, "hadamard", 2, 1),
    (4, 4, "hadamard", 2, 1), (1, 2, "none", 1, 1), (4, 2, "perm", 2, 1),
    (4, 2, "hadamard", 2, 4), (4, 2, "hadamard", 5, 1), (2, 1, "hadamard", 1, 2),
    (4, 2, "dense", 4, 4), (1, 4, "dense", 4, 1), (2, 1, "dense", 4, 1), (4, 1, "perm", 2, 1)])
def test_decode_bits(kbits, vbits, rot, cid, G):
    """b-bit decode (the kernel for widths other than 2/2) against the
    oracle on the same cache bytes: keys and values at their own widths,
    none / Hadamard / reordered Hadamard, a query group, fp16 sinks and
    residual tokens (LLaMA-2-13B recipe), a ragged INT2 range that starts
    inside a tile and spans several tiles and splits."""
    T = 900
    extra = dict(t_new=0) if cid == 4 else {}
    cfg = W.small_config(W.config(cid), T=T, B=2, Hkv=2, Hq=2 * G, **extra)
    perm = (W.channel_orders(cfg) if rot == "perm" else
            W.dense_rotations(cfg) if rot == "dense" else None)
    Rm = rot_matrix(rot, perm)
    K = W.kv_tokens(cfg, "K")
    V = W.kv_tokens(cfg, "V")
    kh = K.permute(0, 2, 1, 3).contiguous().numpy()
    vh = V.permute(0, 2, 1, 3).contiguous().numpy()
    kcache = O.quantize_cache(kh, Rm, bits=kbits)
    vcache = O.quantize_cache(vh, Rm, bits=vbits)
    q = W.queries(cfg)
    fp16 = {}
    tb, te = (cfg.n_sink, T - cfg.n_res) if (cfg.n_sink or cfg.n_res) else (7, T - 5)
    if cfg.n_sink or cfg.n_res:
        fp16 = dict(sink_k=np.ascontiguousarray(kh[:, :, :cfg.n_sink]).astype(np.float16),
                    sink_v=np.ascontiguousarray(vh[:, :, :cfg.n_sink]).astype(np.float16),
                    res_k=np.ascontiguousarray(kh[:, :, T - cfg.n_res:]).astype(np.float16),
                    res_v=np.ascontiguousarray(vh[:, :, T - cfg.n_res:]).astype(np.float16))
    up = {k: torch.from_numpy(v).to(DEV) for k, v in fp16.items()}
    out = kvq.kvq_decode_attention(q.to(DEV), cache_from_numpy(*kcache), cache_from_numpy(*vcache),
                                   tb, te, rot=rot, R=_rot_arg(rot, perm), **up)
    torch.cuda.synchronize()
    ref = O.decode_attention(q.numpy(), kcache, vcache, tb, te, Rm, **fp16)
    err = normwise_rel_err(out.float().cpu().numpy(), ref)
    _report(f"decode bits K{kbits}V{vbits} {rot} c{cid} G={G}", normwise=err)
    assert err <= ATTN_TOL


@pytest.mark.parametrize("kbits,vbits,rot,cid,G", [
    (1, 1, "hadamard", 2, 4), (1, 2, "perm", 2, 2), (1, 4, "dense", 4, 8), (2, 1, "none", 1, 3),
    (2, 4, "hadamard", 5, 4), (4, 1, "hadamard", 2, 2), (4, 2, "perm", 2, 8), (4, 4, "dense", 4, 4),
    (4, 4, "hadamard", 2, 3)])
def test_decode_bits_gqa(kbits, vbits, rot, cid, G):
    """Grouped-query decode at widths other than 2/2 (the matrix-core b-bit
    kernel: 1-bit keys as four shifted copies, 1-bit values spread to 2-bit
    fields, 4-bit codes as two 2-bit planes) against the oracle on the same
    cache bytes: every width pair,
    query groups of 2, 3 (a partial group of four heads), 4 and 8 (two
    groups), every rotation, fp16 sinks and residual tokens (LLaMA-2-13B
    recipe), a ragged INT2 range that starts inside a tile."""
    T = 900
    extra = dict(t_new=0) if cid == 4 else {}
    cfg = W.small_config(W.config(cid), T=T, B=2, Hkv=2, Hq=2 * G, **extra)
    perm = (W.channel_orders(cfg) if rot == "perm" else
            W.dense_rotations(cfg) if rot == "dense" else None)
    Rm = rot_matrix(rot, perm)
    kh = W.kv_tokens(cfg, "K").permute(0, 2, 1, 3).contiguous().numpy()
    vh = W.kv_tokens(cfg, "V").permute(0, 2, 1, 3).contiguous().numpy()
    kcache = O.quantize_cache(kh, Rm, bits=kbits)
    vcache = O.quantize_cache(vh, Rm, bits=vbits)
    q = W.queries(cfg)
    fp16 = {}
    tb, te = (cfg.n_sink, T - cfg.n_res) if (cfg.n_sink or cfg.n_res) else (7, T - 5)
    if cfg.n_sink or cfg.n_res:
        fp16 = dict(sink_k=np.ascontiguousarray(kh[:, :, :cfg.n_sink]).astype(np.float16),
                    sink_v=np.ascontiguousarray(vh[:, :, :cfg.n_sink]).astype(np.float16),
                    res_k=np.ascontiguousarray(kh[:, :, T - cfg.n_res:]).astype(np.float16),
                    res_v=np.ascontiguousarray(vh[:, :, T - cfg.n_res:]).astype(np.float16))
    up = {k: torch.from_numpy(v).to(DEV) for k, v in fp16.items()}
    out = kvq.kvq_decode_attention(q.to(DEV), cache_from_numpy(*kcache), cache_from_numpy(*vcache),
                                   tb, te, rot=rot, R=_rot_arg(rot, perm), **up)
    torch.cuda.synchronize()
    ref = O.decode_attention(q.numpy(), kcache, vcache, tb, te, Rm, **fp16)
    err = normwise_rel_err(out.float().cpu().numpy(), ref)
    _report(f"decode bits gqa K{kbits}V{vbits} {rot} c{cid} G={G}", normwise=err)
    assert err <= ATTN_TOL
    if fp16:                                   # the INT2 part alone (the x50 sinks dominate)
        out2 = kvq.kvq_decode_attention(q.to(DEV), cache_from_numpy(*kcache), cache_from_numpy(*vcache),
                                        tb, te, rot=rot, R=_rot_arg(rot, perm))
        torch.cuda.synchronize()
        ref2 = O.decode_attention(q.numpy(), kcache, vcache, tb, te, Rm)
        err2 = normwise_rel_err(out2.float().cpu().numpy(), ref2)
        _report(f"decode bits gqa K{kbits}V{vbits} INT2 only", normwise=err2)
        assert err2 <= ATTN_TOL


@pytest.mark.parametrize("kbits,vbits,rot,cid,G,P", [
    (4, 2, "hadamard", 2, 1, 128), (1, 4, "perm", 2, 2, 64), (2, 1, "hadamard", 5, 1, 64),
    (4, 1, "dense", 4, 4, 64)])
def test_decode_bits_varlen_paged(kbits, vbits, rot, cid, G, P):
    """b-bit decode with per-sequence ends, over a contiguous cache
    (kvq_decode_attention_varlen_bits) and over a paged one (block table
    over a shuffled pool): each sequence against the oracle on the same
    rows, and the two layouts against each other.  Ends: the full range,
    a ragged one and one just past the first tile."""
    T = 768
    extra = dict(t_new=0) if cid == 4 else {}
    cfg = W.small_config(W.config(cid), T=T, B=3, Hkv=2, Hq=2 * G, **extra)
    rng = np.random.default_rng(300 + kbits * 10 + vbits)
    perm = (W.channel_orders(cfg) if rot == "perm" else
            W.dense_rotations(cfg) if rot == "dense" else None)
    Rm = rot_matrix(rot, perm)
    kh = W.kv_tokens(cfg, "K").permute(0, 2, 1, 3).contiguous().numpy()
    vh = W.kv_tokens(cfg, "V").permute(0, 2, 1, 3).contiguous().numpy()
    kcache = O.quantize_cache(kh, Rm, bits=kbits)
    vcache = O.quantize_cache(vh, Rm, bits=vbits)
    table, n_pages = _page_layout(rng, cfg.B, T, P)
    te_max = T - cfg.n_res
    tb = cfg.n_sink if cfg.n_sink else 5
    ends = np.array([te_max, tb + 1 + int(rng.integers(0, te_max - tb - 1)), tb + 64 + 3], np.int32)
    fp16 = {}
    if cfg.n_sink or cfg.n_res:
        fp16 = dict(sink_k=np.ascontiguousarray(kh[:, :, :cfg.n_sink]).astype(np.float16),
                    sink_v=np.ascontiguousarray(vh[:, :, :cfg.n_sink]).astype(np.float16),
                    res_k=np.ascontiguousarray(kh[:, :, T - cfg.n_res:]).astype(np.float16),
                    res_v=np.ascontiguousarray(vh[:, :, T - cfg.n_res:]).astype(np.float16))
    up = {k: torch.from_numpy(v).to(DEV) for k, v in fp16.items()}
    kp = kvq.PagedCache(*[torch.from_numpy(a).to(DEV) for a in _to_pages(kcache, table, n_pages, P)])
    vp = kvq.PagedCache(*[torch.from_numpy(a).to(DEV) for a in _to_pages(vcache, table, n_pages, P)])
    assert (kp.bits, vp.bits) == (kbits, vbits)
    q = W.queries(cfg)
    tends = torch.from_numpy(ends).to(DEV)
    Rg = _rot_arg(rot, perm)
    out = kvq.kvq_decode_attention_paged(q.to(DEV), kp, vp, tb, tends, te_max,
                                         torch.from_numpy(table).to(DEV), rot=rot, R=Rg, **up)
    flat = kvq.kvq_decode_attention(q.to(DEV), cache_from_numpy(*kcache), cache_from_numpy(*vcache),
                                    tb, te_max, rot=rot, R=Rg, t_ends=tends, **up)
    torch.cuda.synchronize()
    out, flat = out.float().cpu().numpy(), flat.float().cpu().numpy()
    worst = worst_flat = 0.0
    for b in range(cfg.B):
        sl = lambda c: tuple(a[b:b + 1] for a in c)
        kwb = {k: v[b:b + 1] for k, v in fp16.items()}
        ref = O.decode_attention(q.numpy()[b:b + 1], sl(kcache), sl(vcache), tb, int(ends[b]), Rm, **kwb)
        worst = max(worst, normwise_rel_err(out[b:b + 1], ref))
        worst_flat = max(worst_flat, normwise_rel_err(flat[b:b + 1], ref))
    err = normwise_rel_err(out, flat)
    _report(f"decode bits varlen/paged K{kbits}V{vbits} {rot} c{cid} G={G} P={P}",
            paged=worst, contiguous=worst_flat, paged_vs_contiguous=err)
    assert worst <= ATTN_TOL and worst_flat <= ATTN_TOL and err <= 1e-3


@pytest.mark.parametrize("kbits,vbits,rot,Hkv,P", [(4, 2, "hadamard", 4, 128), (1, 4, "perm", 3, 64),
                                                   (4, 1, "dense", 2, 64)])
def test_quantize_bits_varlen_paged(kbits, vbits, rot, Hkv, P):
    """b-bit writes at per-sequence slots: the contiguous write
    (kvq_quantize_at_bits) against the oracle's codec at rounding ties, with
    the slots outside each sequence's rows left untouched; the paged write
    of the same rows bit for bit equal to it, and nothing else in the pool
    touched."""
    cfg = W.small_config(W.config(2), B=3, T=150, Hkv=Hkv, Hq=Hkv)
    perm = (W.channel_orders(cfg) if rot == "perm" else
            W.dense_rotations(cfg) if rot == "dense" else None)
    Rm = rot_matrix(rot, perm)
    Rg = _rot_arg(rot, perm)
    rng = np.random.default_rng(9)
    T_cap = 4 * P
    table, n_pages = _page_layout(rng, cfg.B, T_cap, P)
    offs = np.array([0, 37, P - 20], np.int32)
    toffs = torch.from_numpy(offs).to(DEV)
    K, V = W.kv_tokens(cfg, "K"), W.kv_tokens(cfg, "V")
    kc = empty_cache(cfg.B, Hkv, T_cap, bits=kbits)
    vc = empty_cache(cfg.B, Hkv, T_cap, bits=vbits)
    kvq.kvq_quantize(K.to(DEV), V.to(DEV), kc, vc, rot=rot, R=Rg, t_offsets=toffs)
    pk = kvq.PagedCache.empty(n_pages, Hkv, P, bits=kbits)
    pv = kvq.PagedCache.empty(n_pages, Hkv, P, bits=vbits)
    for c in (pk, pv):
        for t in (c.codes, c.scales.view(torch.uint8), c.zeros.view(torch.uint8)):
            t.fill_(SENTINEL)
    kvq.kvq_quantize_paged(K.to(DEV), V.to(DEV), pk, pv, toffs, torch.from_numpy(table).to(DEV),
                           rot=rot, R=Rg)
    torch.cuda.synchronize()
    tot = dict(elements=0, code_mismatch=0, group_scale_zero_diff=0)
    for x, c, p_c, bits in ((K, kc, pk, kbits), (V, vc, pv, vbits)):
        fc, pc = cache_to_numpy(c), cache_to_numpy(p_c)
        xh = x.permute(0, 2, 1, 3).contiguous().numpy()
        ora = O.quantize_cache(xh, Rm, bits=bits)
        written = np.zeros((n_pages, P), bool)
        for b in range(cfg.B):
            o = int(offs[b])
            for arr in (fc[0], fc[1].view(np.uint8), fc[2].view(np.uint8)):
                assert np.all(arr[b, :, :o] == SENTINEL) and np.all(arr[b, :, o + cfg.T:] == SENTINEL)
            for h in range(Hkv):
                Rh = Rm[h] if rot in ("perm", "dense") else Rm
                st = compare_codes_at_ties(xh[b:b + 1, h], Rh,
                                           tuple(a[b:b + 1, h, o:o + cfg.T] for a in fc),
                                           tuple(a[b:b + 1, h] for a in ora), max_frac=1.0, bits=bits)
                for k in tot:
                    tot[k] += st[k]
            for t in range(cfg.T):
                slot = o + t
                page = int(table[b, slot // P])
                written[page, slot % P] = True
                for a_p, a_f in zip(pc, fc):
                    assert np.array_equal(a_p[page, :, slot % P].view(np.uint8),
                                          a_f[b, :, slot].view(np.uint8))
        for a_p in pc:
            assert np.all(np.moveaxis(a_p.view(np.uint8), 1, 2)[~written] == SENTINEL)
    _report(f"quantize bits varlen/paged K{kbits}V{vbits} {rot} P={P}", **tot)
    assert tot["code_mismatch"] <= 1e-5 * tot["elements"]


@pytest.mark.parametrize("B,Hq,kbits,vbits", [(64, 1, 2, 2), (70, 1, 2, 2), (67, 4, 2, 2), (130, 1, 2, 2),
                                              (70, 1, 4, 2), (130, 2, 1, 4)])
def test_decode_varlen_many_sequences(B, Hq, kbits, vbits):
    """Variable-length batches of many sequences with a skewed length mix:
    one sequence spans the whole range, the rest are short or empty.  The
    attention waves are shared among the sequences by tile count, so this
    covers batches of one wave's width (64) and wider ones, for one query
    head per KV head and for a query group, and at other code widths (the
    b-bit kernel takes the same wave map).

    Checks: (1) each sequence's output matches a one-sequence call over the
    same range (which other tests hold to the oracle), so every sequence
    got exactly its own tiles; (2) against the oracle, the error relative to
    the largest attended value row.  A short range's output can be far
    smaller than the rows it averages (they cancel), so the per-row
    normwise reading would measure the cancellation, not the arithmetic,
    whose error scales with the value rows."""
    T = 1300
    cfg = W.small_config(W.config(1), T=T, B=B, Hkv=1, Hq=Hq)
    tb, te_max = 5, T
    rng = np.random.default_rng(1000 + B)
    ends = (tb + rng.integers(0, 200, B)).astype(np.int32)
    ends[rng.random(B) < 0.2] = tb                         # empty sequences
    ends[B // 3] = te_max                                  # one long sequence
    K = W.kv_tokens(cfg, "K")
    V = W.kv_tokens(cfg, "V")
    kh = K.permute(0, 2, 1, 3).contiguous().numpy()
    vh = V.permute(0, 2, 1, 3).contiguous().numpy()
    Rm = rot_matrix("hadamard", None)
    kcache = O.quantize_cache(kh, Rm, bits=kbits)
    vcache = O.quantize_cache(vh, Rm, bits=vbits)
    q = W.queries(cfg)
    out = kvq.kvq_decode_attention(q.to(DEV), cache_from_numpy(*kcache), cache_from_numpy(*vcache),
                                   tb, te_max, rot="hadamard", t_ends=torch.from_numpy(ends).to(DEV))
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    worst_single, worst_oracle = 0.0, 0.0
    for b in range(B):
        if ends[b] == tb:
            assert np.all(out[b] == 0.0)                   # no token at all: zero output
            continue
        sl = lambda c: tuple(a[b:b + 1] for a in c)
        one = kvq.kvq_decode_attention(q[b:b + 1].to(DEV), cache_from_numpy(*sl(kcache)),
                                       cache_from_numpy(*sl(vcache)), tb, int(ends[b]), rot="hadamard")
        torch.cuda.synchronize()
        worst_single = max(worst_single, normwise_rel_err(out[b:b + 1], one.float().cpu().numpy()))
        ref = O.decode_attention(q.numpy()[b:b + 1], sl(kcache), sl(vcache), tb, int(ends[b]), Rm)
        vrows = O.dequantize(O.unpack_codes(vcache[0][b, 0, tb:ends[b]], vbits), vcache[1][b, 0, tb:ends[b]],
                             vcache[2][b, 0, tb:ends[b]]) @ Rm.T          # attended rows, original basis
        worst_oracle = max(worst_oracle, float(np.abs(out[b] - ref[0]).max() / np.abs(vrows).max()))
    _report(f"decode varlen B={B} Hq={Hq} K{kbits}V{vbits}", vs_single=worst_single,
            vs_oracle_value_scale=worst_oracle)
    assert worst_single <= 1e-4
    assert worst_oracle <= ATTN_TOL


@pytest.mark.parametrize("rot,bits", [("none", 2), ("hadamard", 2), ("perm", 2), ("dense", 2),
                                      ("dense", 1), ("dense", 4), ("perm", 4)])
def test_quantize_at_per_sequence_slots(rot, bits):
    """kvq_quantize_at (kvq_quantize_at_bits at 1 and 4 bits): each
    sequence's new rows land at its own slot; rows whose slot falls outside
    [0, T_cap) are skipped and every other slot keeps its sentinel bytes.
    T_new = 1 (a decode-step append) and T_new = 5."""
    T_cap = 40
    cfg = W.small_config(W.config(2), B=4, T=5, Hkv=2, Hq=2)
    R = W.dense_rotations(cfg) if rot == "dense" else (
        np.stack([np.random.default_rng(4).permutation(128) for _ in range(cfg.Hkv)]).astype(np.int32)
        if rot == "perm" else None)
    Rm = rot_matrix(rot, R)
    for T_new, offs in ((1, [0, 17, 39, 25]), (5, [3, 37, -2, 20])):
        x = W.kv_tokens(cfg, "K")[:, :T_new]                      # [B, T_new, H, d] fp16
        c = empty_cache(cfg.B, cfg.Hkv, T_cap, bits=bits)
        offsets = torch.tensor(offs, dtype=torch.int32, device=DEV)
        kvq.kvq_quantize(x.to(DEV), None, c, None, rot=rot, R=_rot_arg(rot, R), t_offsets=offsets)
        torch.cuda.synchronize()
        gp, gs, gz = cache_to_numpy(c)
        op, os_, oz = _oracle_quantize(x, rot, R, bits)           # [B, H, T_new, ...]
        xr = x.permute(0, 2, 1, 3).contiguous().numpy()
        for b in range(cfg.B):
            written = np.zeros(T_cap, bool)
            for t in range(T_new):
                slot = offs[b] + t
                if not 0 <= slot < T_cap:
                    continue
                written[slot] = True
                g = (gp[b, :, slot:slot + 1], gs[b, :, slot:slot + 1], gz[b, :, slot:slot + 1])
                o = (op[b, :, t:t + 1], os_[b, :, t:t + 1], oz[b, :, t:t + 1])
                if rot == "none":
                    assert np.array_equal(g[0], o[0])
                    assert np.array_equal(g[1].view(np.uint16), o[1].view(np.uint16))
                    assert np.array_equal(g[2].view(np.uint16), o[2].view(np.uint16))
                else:
                    for h in range(cfg.Hkv):
                        Rh = Rm[h] if (rot != "hadamard" and np.asarray(Rm).ndim == 3) else Rm
                        compare_codes_at_ties(xr[b, h, t:t + 1], Rh, tuple(a[h] for a in g),
                                              tuple(a[h] for a in o), max_frac=1.0, bits=bits)
            for arr in (gp, gs.view(np.uint8), gz.view(np.uint8)):
                assert np.all(arr[b][:, ~written] == SENTINEL)
        _report(f"quantize_at {rot} bits={bits} T_new={T_new}", offsets=offs)


# ---------------------------------------------------------- end to end
def test_end_to_end_dense_gqa():
    """Dense rotation, GQA group 4: GPU quantize (MFMA) -> GPU decode, against
    the oracle decode on the GPU's own codes."""
    cfg = W.small_config(W.config(4), B=2, T=1500, Hkv=2, Hq=8, t_new=0)
    R = W.dense_rotations(cfg)
    Rg = torch.as_tensor(R, device=DEV).contiguous()
    K = W.kv_tokens(cfg, "K").to(DEV)
    V = W.kv_tokens(cfg, "V").to(DEV)
    ck, cv = empty_cache(cfg.B, cfg.Hkv, cfg.T), empty_cache(cfg.B, cfg.Hkv, cfg.T)
    kvq.kvq_quantize(K, V, ck, cv, rot="dense", R=Rg)
    q = W.queries(cfg).to(DEV)
    out = kvq.kvq_decode_attention(q, ck, cv, 0, cfg.T, rot="dense", R=Rg)
    torch.cuda.synchronize()
    gk, gv = cache_to_numpy(ck), cache_to_numpy(cv)
    ref = O.decode_attention(q.cpu().numpy(), gk, gv, 0, cfg.T, R)
    err = normwise_rel_err(out.float().cpu().numpy(), ref)
    _report("end_to_end dense G=4", normwise=err)
    assert err <= ATTN_TOL


@pytest.mark.parametrize("cid", [1, 2])
def test_end_to_end_gpu_codes(cid):
    """GPU quantize -> GPU decode, against the oracle decode on the GPU's own
    codes; the GPU codes themselves are checked against the oracle's."""
    cfg = W.config(cid)
    K = W.kv_tokens(cfg, "K").to(DEV)
    V = W.kv_tokens(cfg, "V").to(DEV)
    ck = empty_cache(cfg.B, cfg.Hkv, cfg.T)
    cv = empty_cache(cfg.B, cfg.Hkv, cfg.T)
    kvq.kvq_quantize(K, V, ck, cv, rot="hadamard")
    q = W.queries(cfg).to(DEV)
    out = kvq.kvq_decode_attention(q, ck, cv, 0, cfg.T, rot="hadamard")
    torch.cuda.synchronize()
    H = rot_matrix("hadamard")
    gk, gv = cache_to_numpy(ck), cache_to_numpy(cv)
    for x, g in ((K, gk), (V, gv)):
        xr = x.cpu().permute(0, 2, 1, 3).contiguous().numpy()
        compare_codes_at_ties(xr, H, g, O.quantize_cache(xr, H))
    ref = O.decode_attention(q.cpu().numpy(), gk, gv, 0, cfg.T, H)
    err = normwise_rel_err(out.float().cpu().numpy(), ref)
    _report(f"end_to_end c{cid}", normwise=err)
    assert err <= ATTN_TOL
