"""Parity at the workloads' full sizes, in the launch configuration the
benchmark uses (same shapes, so the same grid and split plan).

The whole cache is written and read on the GPU; the oracle recomputes
sampled (batch, KV head) slices one at a time: the codes of that head must
match at ties, and the decode outputs of the head's query heads must be
within the attention bar against the oracle run on the GPU's own codes of
that head.  The sample's inputs are regenerated on the CPU from the seeded
generator and checked equal to the device copy first.
"""
import json

import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O
import workloads as W
import int2_rotated_kv_amd as kvq
from parity_util import (require_gpu, rot_matrix, compare_codes_at_ties, normwise_rel_err)

pytestmark = pytest.mark.gpu
DEV = "cuda"
ATTN_TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def _report(name, **kw):
    print(f"[fullsize] {name} " + json.dumps(kw), flush=True)


def _head_slice_cpu(cfg, which, b, h, t0=0, t1=None):
    """[T, d] rows of (batch b, KV head h) regenerated on the CPU."""
    return W.kv_tokens(cfg, which, b0=b, b1=b + 1, h0=h, h1=h + 1, t0=t0, t1=t1)[0, :, 0]


def _contiguous_head(c, b, hk):
    """(codes, scales, zeros) of head (b, hk) of a contiguous cache side, [T, ...]."""
    return tuple(a[b, hk] for a in (c.codes, c.scales, c.zeros))


# Scale/zero groups that may differ by one fp16 ulp (each only at an fp16
# rounding boundary of the exact value, which compare_codes_at_ties checks):
# the rounding of the fp32 Hadamard transform moves about 6e-5 of the groups
# of these workloads across a boundary, the fp16 hi/lo split of a dense R
# about 5e-4 (both measured by emulating the transform in numpy float32).
GROUP_RATE = {"hadamard": 1e-4, "perm": 1e-4, "dense": 1e-3}


class GroupTally:
    """Scale/zero mismatches over the sampled heads of one test."""

    def __init__(self, rot):
        self.rot, self.diff, self.groups = rot, 0, 0

    def add(self, stats):
        for side in stats.values():
            self.diff += side["group_scale_zero_diff"]
            self.groups += side["groups"]

    def check(self, name):
        rate = self.diff / max(self.groups, 1)
        _report(f"{name} scale/zero group mismatch", rate=rate, groups=self.groups)
        assert rate <= GROUP_RATE[self.rot], f"scale/zero mismatch rate {rate:.3g}"


def _check_head(cfg, Kd, Vd, ck, cv, out, q, b, hk, rot, R, t_begin, t_end,
                sink=None, res=None, code_end=None, head_rows=_contiguous_head):
    """Codes of head (b, hk) vs oracle at ties (rows [t_begin, code_end),
    default t_end); decode of its query heads over [t_begin, t_end) vs the
    oracle on the GPU codes.  Each cache side is read at its own width;
    head_rows(side, b, hk) gives the head's rows in token order."""
    code_end = t_end if code_end is None else code_end
    kh, vh = head_rows(ck, b, hk), head_rows(cv, b, hk)
    Rm = rot_matrix(rot, R)
    Rh = Rm if rot != "dense" else Rm[hk]
    stats = {}
    for which, xd, c, rows in (("K", Kd, ck, kh), ("V", Vd, cv, vh)):
        x_cpu = _head_slice_cpu(cfg, which, b, hk)
        x_dev = xd[b, :, hk].cpu()
        assert torch.equal(x_cpu, x_dev), "generator differs between CPU and GPU"
        xr = x_cpu[t_begin:code_end].numpy()[None]             # [1, T, d]
        gpu = tuple(a[t_begin:code_end].cpu().numpy()[None] for a in rows)
        ora = O.quantize_cache(xr[:, None], Rh, bits=c.bits)
        ora = tuple(a[:, 0] for a in ora)
        stats[which] = compare_codes_at_ties(xr, Rh, gpu, ora, bits=c.bits)
    G = cfg.G
    hq = slice(hk * G, hk * G + G)
    kc = tuple(a.cpu().numpy()[None, None] for a in kh)
    vc = tuple(a.cpu().numpy()[None, None] for a in vh)
    kw = {}
    if sink is not None:
        kw.update(sink_k=sink[0][b:b + 1, hk:hk + 1].cpu().numpy(),
                  sink_v=sink[1][b:b + 1, hk:hk + 1].cpu().numpy())
    if res is not None:
        kw.update(res_k=res[0][b:b + 1, hk:hk + 1].cpu().numpy(),
                  res_v=res[1][b:b + 1, hk:hk + 1].cpu().numpy())
    Rd = Rh if Rh is None or rot != "dense" else Rh[None]
    ref = O.decode_attention(q[b:b + 1, hq].cpu().numpy(), kc, vc, t_begin, t_end, Rd, **kw)
    err = normwise_rel_err(out[b:b + 1, hq].float().cpu().numpy(), ref)
    return stats, err


def test_fullsize_config3_throughput():
    cfg = W.config(3)
    B, T, H, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    K = W.kv_tokens(cfg, "K", device=DEV)
    V = W.kv_tokens(cfg, "V", device=DEV)
    q = W.queries(cfg, device=DEV)
    ck, cv = kvq.Int2Cache.empty(B, H, T), kvq.Int2Cache.empty(B, H, T)
    kvq.kvq_quantize(K, V, ck, cv, rot="hadamard")
    out = kvq.kvq_decode_attention(q, ck, cv, 0, T, rot="hadamard")
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    tally = GroupTally("hadamard")
    for b, hk in ((0, 0), (7, 13), (15, 31)):
        stats, err = _check_head(cfg, K, V, ck, cv, out, q, b, hk, "hadamard", None, 0, T)
        _report(f"c3 b={b} h={hk}", normwise=err, K=stats["K"], V=stats["V"])
        tally.add(stats)
        assert err <= ATTN_TOL
    tally.check("c3")


def test_fullsize_config4_dense_gqa():
    cfg = W.config(4)
    B, T, H, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    R = W.dense_rotations(cfg)
    Rg = torch.as_tensor(R, device=DEV).contiguous()
    K = W.kv_tokens(cfg, "K", device=DEV)
    V = W.kv_tokens(cfg, "V", device=DEV)
    q = W.queries(cfg, device=DEV)
    ck, cv = kvq.Int2Cache.empty(B, H, T), kvq.Int2Cache.empty(B, H, T)
    p0, p1 = cfg.quant_range                     # prefill slice [98304, 131072)
    kvq.kvq_quantize(K[:, :p0], V[:, :p0], ck, cv, rot="dense", R=Rg)
    kvq.kvq_quantize(K[:, p0:p1], V[:, p0:p1], ck, cv, rot="dense", R=Rg, t_offset=p0)
    out = kvq.kvq_decode_attention(q, ck, cv, 0, T, rot="dense", R=Rg)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    tally = GroupTally("dense")
    for b, hk in ((0, 0), (3, 5)):
        stats, err = _check_head(cfg, K, V, ck, cv, out, q, b, hk, "dense", R, 0, T)
        _report(f"c4 b={b} h={hk}", normwise=err, K=stats["K"], V=stats["V"])
        tally.add(stats)
        assert err <= ATTN_TOL
    tally.check("c4")


def test_fullsize_config5_sinks_residual():
    cfg = W.config(5)
    B, T, H, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    tb, te = cfg.int2_range                     # [4, 65408)
    K = W.kv_tokens(cfg, "K", device=DEV)
    V = W.kv_tokens(cfg, "V", device=DEV)
    q = W.queries(cfg, device=DEV)
    ck, cv = kvq.Int2Cache.empty(B, H, T), kvq.Int2Cache.empty(B, H, T)
    kvq.kvq_quantize(K[:, tb:te], V[:, tb:te], ck, cv, rot="hadamard", t_offset=tb)
    sink = tuple(x[:, :tb].permute(0, 2, 1, 3).contiguous() for x in (K, V))
    res = tuple(x[:, te:].permute(0, 2, 1, 3).contiguous() for x in (K, V))
    out = kvq.kvq_decode_attention(q, ck, cv, tb, te, rot="hadamard", sink_k=sink[0],
                                   sink_v=sink[1], res_k=res[0], res_v=res[1])
    out_int2 = kvq.kvq_decode_attention(q, ck, cv, tb, te, rot="hadamard")
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(out_int2.float()).all()
    tally = GroupTally("hadamard")
    for b, hk in ((0, 0), (5, 27)):
        stats, err = _check_head(cfg, K, V, ck, cv, out, q, b, hk, "hadamard", None, tb, te,
                                 sink=sink, res=res)
        _, err2 = _check_head(cfg, K, V, ck, cv, out_int2, q, b, hk, "hadamard", None, tb, te)
        _report(f"c5 b={b} h={hk}", normwise_full=err, normwise_int2_only=err2,
                K=stats["K"], V=stats["V"])
        tally.add(stats)
        assert err <= ATTN_TOL and err2 <= ATTN_TOL
    tally.check("c5")


def test_fullsize_config3_key4_value2():
    """Throughput shapes with 4-bit keys and 2-bit values (the b-bit write
    and decode kernels, as bench.py --kbits 4 --vbits 2 runs them)."""
    cfg = W.config(3)
    B, T, H, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    K = W.kv_tokens(cfg, "K", device=DEV)
    V = W.kv_tokens(cfg, "V", device=DEV)
    q = W.queries(cfg, device=DEV)
    ck, cv = kvq.Int2Cache.empty(B, H, T, bits=4), kvq.Int2Cache.empty(B, H, T, bits=2)
    kvq.kvq_quantize(K, V, ck, cv, rot="hadamard")
    out = kvq.kvq_decode_attention(q, ck, cv, 0, T, rot="hadamard")
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    tally = GroupTally("hadamard")
    for b, hk in ((0, 0), (9, 17)):
        stats, err = _check_head(cfg, K, V, ck, cv, out, q, b, hk, "hadamard", None, 0, T)
        _report(f"c3 K4V2 b={b} h={hk}", normwise=err, K=stats["K"], V=stats["V"])
        tally.add(stats)
        assert err <= ATTN_TOL
    tally.check("c3 K4V2")


def test_fullsize_config3_key1_value1():
    """Throughput shapes at 1-bit keys and values (bench.py --kbits 1
    --vbits 1): the one-head b-bit decode with its matrix-core key scores and
    value step at the workload's grid and split plan."""
    cfg = W.config(3)
    B, T, H, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    K = W.kv_tokens(cfg, "K", device=DEV)
    V = W.kv_tokens(cfg, "V", device=DEV)
    q = W.queries(cfg, device=DEV)
    ck, cv = kvq.Int2Cache.empty(B, H, T, bits=1), kvq.Int2Cache.empty(B, H, T, bits=1)
    kvq.kvq_quantize(K, V, ck, cv, rot="hadamard")
    out = kvq.kvq_decode_attention(q, ck, cv, 0, T, rot="hadamard")
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    tally = GroupTally("hadamard")
    for b, hk in ((0, 0), (13, 30)):
        stats, err = _check_head(cfg, K, V, ck, cv, out, q, b, hk, "hadamard", None, 0, T)
        _report(f"c3 K1V1 b={b} h={hk}", normwise=err, K=stats["K"], V=stats["V"])
        tally.add(stats)
        assert err <= ATTN_TOL
    tally.check("c3 K1V1")


def test_fullsize_config3_varlen():
    """Throughput shapes as a mixed-length batch (the ends bench.py --varlen
    draws): sampled sequences against the oracle over their own ranges."""
    cfg = W.config(3)
    B, T, H, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    K = W.kv_tokens(cfg, "K", device=DEV)
    V = W.kv_tokens(cfg, "V", device=DEV)
    q = W.queries(cfg, device=DEV)
    ck, cv = kvq.Int2Cache.empty(B, H, T), kvq.Int2Cache.empty(B, H, T)
    kvq.kvq_quantize(K, V, ck, cv, rot="hadamard")
    rng = np.random.default_rng(np.random.SeedSequence([1000 + cfg.cid, 77]))
    ends = rng.integers(T // 2, T + 1, size=B).astype(np.int32)
    out = kvq.kvq_decode_attention(q, ck, cv, 0, T, rot="hadamard",
                                   t_ends=torch.from_numpy(ends).to(DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    for b, hk in ((int(np.argmin(ends)), 3), (int(np.argmax(ends)), 30), (5, 11)):
        _, err = _check_head(cfg, K, V, ck, cv, out, q, b, hk, "hadamard", None, 0, int(ends[b]),
                             code_end=64)
        _report(f"c3 varlen b={b} end={int(ends[b])} h={hk}", normwise=err)
        assert err <= ATTN_TOL


def test_fullsize_config5_paged():
    """LLaMA-2-13B shapes in a paged cache of 128-token pages over a pool
    shuffled per sequence (the table bench.py --config 5 --paged 128 draws):
    the paged write, then the paged decode with sinks and residual tokens;
    sampled heads gathered back through the table against the oracle."""
    cfg = W.config(5)
    B, T, H, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    P = 128
    tb, te = cfg.int2_range
    per = (T + P - 1) // P
    pool = np.random.default_rng(np.random.SeedSequence([2000 + cfg.cid, P])).permutation(B * per)
    table_h = pool.reshape(B, per).astype(np.int32)
    table = torch.from_numpy(table_h).to(DEV)
    K = W.kv_tokens(cfg, "K", device=DEV)
    V = W.kv_tokens(cfg, "V", device=DEV)
    q = W.queries(cfg, device=DEV)
    ck, cv = kvq.PagedCache.empty(B * per, H, P), kvq.PagedCache.empty(B * per, H, P)
    offs = torch.full((B,), tb, dtype=torch.int32, device=DEV)
    kvq.kvq_quantize_paged(K[:, tb:te], V[:, tb:te], ck, cv, offs, table, rot="hadamard")
    sink = tuple(x[:, :tb].permute(0, 2, 1, 3).contiguous() for x in (K, V))
    res = tuple(x[:, te:].permute(0, 2, 1, 3).contiguous() for x in (K, V))
    ends = torch.full((B,), te, dtype=torch.int32, device=DEV)
    out = kvq.kvq_decode_attention_paged(q, ck, cv, tb, ends, te, table, rot="hadamard",
                                         sink_k=sink[0], sink_v=sink[1], res_k=res[0], res_v=res[1])
    # the sinks take most of the weight on these inputs, so the INT2 rows
    # are also checked on their own
    out_int2 = kvq.kvq_decode_attention_paged(q, ck, cv, tb, ends, te, table, rot="hadamard")
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(out_int2.float()).all()
    t = torch.arange(T, device=DEV)

    def paged_head(c, b, hk):
        pages = table[b][t // P].long()
        return tuple(a[pages, hk, t % P] for a in (c.codes, c.scales, c.zeros))

    for b, hk in ((0, 0), (6, 33)):
        stats, err = _check_head(cfg, K, V, ck, cv, out, q, b, hk, "hadamard", None, tb, te,
                                 sink=sink, res=res, head_rows=paged_head)
        _, err2 = _check_head(cfg, K, V, ck, cv, out_int2, q, b, hk, "hadamard", None, tb, te,
                              head_rows=paged_head)
        _report(f"c5 paged P={P} b={b} h={hk}", normwise_full=err, normwise_int2_only=err2,
                K=stats["K"], V=stats["V"])
        assert err <= ATTN_TOL and err2 <= ATTN_TOL


def test_fullsize_config4_dense_gqa_key4_value2():
    """GQA shapes with a dense R at 4-bit keys and 2-bit values (the dense
    write kernel at two widths and the b-bit decode over the prepared dense
    query, as bench.py --config 4 --kbits 4 --vbits 2 runs them)."""
    cfg = W.config(4)
    B, T, H, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    R = W.dense_rotations(cfg)
    Rg = torch.as_tensor(R, device=DEV).contiguous()
    K = W.kv_tokens(cfg, "K", device=DEV)
    V = W.kv_tokens(cfg, "V", device=DEV)
    q = W.queries(cfg, device=DEV)
    ck, cv = kvq.Int2Cache.empty(B, H, T, bits=4), kvq.Int2Cache.empty(B, H, T, bits=2)
    p0, p1 = cfg.quant_range
    kvq.kvq_quantize(K[:, :p0], V[:, :p0], ck, cv, rot="dense", R=Rg)
    kvq.kvq_quantize(K[:, p0:p1], V[:, p0:p1], ck, cv, rot="dense", R=Rg, t_offset=p0)
    out = kvq.kvq_decode_attention(q, ck, cv, 0, T, rot="dense", R=Rg)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    tally = GroupTally("dense")
    for b, hk in ((1, 2), (3, 7)):
        stats, err = _check_head(cfg, K, V, ck, cv, out, q, b, hk, "dense", R, 0, T)
        _report(f"c4 K4V2 b={b} h={hk}", normwise=err, K=stats["K"], V=stats["V"])
        tally.add(stats)
        assert err <= ATTN_TOL
    tally.check("c4 K4V2")
