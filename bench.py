#!/usr/bin/env python3
"""Benchmark of the rotated INT2 KV-cache hot path on one MI355X.

One step = the whole path over one batch of the workload (default: the
throughput case B=16, T=32768, 32 heads, d=128, fp16 K/V, Hadamard rotation,
group 32):
  1. kvq_quantize: rotate + quantize + pack the K and V rows of the timed
     token range into the cache;
  2. kvq_decode_attention: one decode query per (batch, query head) over the
     cache (query rotation, split-K attention, merge, un-rotation, fp16
     sink / residual tokens when the workload has them).
The quantize and the decode calls are timed separately: the K quantize
calls run back to back, then the K decode calls (each call bracketed by
events, with an untimed 1 GiB read before each call to evict the caches).
Each timed phase follows about 30 ms of untimed calls of the same kind, so
it is measured in its own steady state.  ms_per_step is the time of one
timed quantize call plus one timed decode call (mean over the steps).  Inputs are generated on the GPU before timing (seeded, synthetic)
and are resident in HBM when the timed region starts.

Prints ONE JSON line.  `value` is the decode attention's effective HBM
bandwidth (algorithmic bytes / time of the decode call); the quantize
throughput, per-kernel rooflines and the oracle's CPU throughput on a
bounded sample are extra fields.  --config 4 (GQA, dense rotation, prefill
slice) and --config 5 (13B-shaped, fp16 sinks and residual) give the same
line for those workloads; the default invocation also runs both as child
processes and summarizes them under other_workloads (--headline-only skips
that).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "INT2 decode attention effective HBM GB/s (% of peak) + quantize tokens/s"

# algorithmic bytes (fp16 K/V input)


def row_bytes(bits):
    """Bytes of one cached row at `bits` per code: 16*bits code bytes plus
    four fp16 scales and four fp16 zeros (48 for INT2)."""
    return 16 * bits + 16


# Algorithmic bytes per (token, KV head): the write reads the fp16 K and V
# rows and writes two cache rows (608 at 2 bits); the decode reads one K and
# one V cache row (96 at 2 bits).
QUANT_BYTES_PER_TOKEN_HEAD = 2 * 256 + 2 * row_bytes(2)
DECODE_BYTES_PER_TOKEN_HEAD = 2 * row_bytes(2)
FP16_BYTES_PER_TOKEN_HEAD = 2 * 256               # read one fp16 K row and one V row


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--perm", action="store_true",
                   help="reordered Hadamard rotation (each head's channels sorted by outlier "
                        "magnitude ahead of the transform) on a Hadamard workload")
    p.add_argument("--varlen", action="store_true",
                   help="serving form: per-sequence lengths drawn in [T/2, T] (seeded); the decode "
                        "is kvq_decode_attention_varlen and the write phase a decode-step append "
                        "of one row per sequence (kvq_quantize_at)")
    p.add_argument("--paged", type=int, default=0, metavar="P",
                   help="keep the cache in pages of P tokens (a multiple of 64) behind a shuffled "
                        "block table (kvq_quantize_paged / kvq_decode_attention_paged)")
    p.add_argument("--kbits", type=int, default=2, choices=(1, 2, 4),
                   help="key code width (1 and 4: the b-bit write and decode kernels)")
    p.add_argument("--vbits", type=int, default=2, choices=(1, 2, 4), help="value code width")
    p.add_argument("--prerope", type=int, default=0, choices=(0, 1, 2, 4), metavar="G",
                   help="keys written before RoPE with the grouped-head rotation over G heads "
                        "(kvq_quantize_prerope / kvq_decode_attention_prerope), on a Hadamard workload")
    p.add_argument("--config", type=int, default=3, choices=(3, 4, 5),
                   help="workload id (3 = throughput case, 4 = GQA dense rotation, 5 = sinks)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--headline-only", action="store_true",
                   help="skip the short child runs of the GQA and LLaMA-2-13B workloads that the default "
                        "invocation adds to its line (other_workloads)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a 1 GiB elementwise device copy (counter calibration)")
    return p.parse_args()


# What the path computes in (the JSON line's "arithmetic" field).
ARITHMETIC_WRITE = "f32 transform of the f16 rows, f32 quantizer (IEEE steps), 2-bit codes + f16 scale/zero"
ARITHMETIC_G1 = {"write": ARITHMETIC_WRITE,
                 "scores": "int32 dot of the codes with a 19-bit fixed-point rotated query, f32 scale/zero terms",
                 "values": "f16 weights p*s times the codes (f16 dot2), f32 accumulation",
                 "combine": "f32 merge and un-rotation, output in the query dtype"}
ARITHMETIC_GQA = {"write": ARITHMETIC_WRITE,
                  "scores": "fp8 digits of a 19-bit fixed-point query x fp4 codes on the matrix cores (exact), "
                            "f32 scale/zero terms",
                  "values": "f16 weights x f16 (code*s - 1.5s) on the matrix cores, f32 accumulation",
                  "combine": "f32 merge and un-rotation, output in the query dtype"}
ARITHMETIC_PREROPE = {"write": ARITHMETIC_WRITE + "; keys rotated over the group's heads",
                      "scores": "exact integer H_32 of the codes on the matrix cores (fp4), f32 scales, butterflies "
                                "over groups and heads, RoPE and dot with the post-RoPE query",
                      "values": "f16 weights p*s times the codes (f16 dot2), f32 accumulation",
                      "combine": "f32 merge and un-rotation, output in the query dtype"}
# Vector ALU issue peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, one fp32
# instruction per lane per cycle (an FMA counts as one operation; packed fp32
# is not used), in tera lane-operations per second
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def prerope_ops_per_unit(gh: int, g: int) -> int:
    """fp32 VALU operations per (INT2 token, KV head) of the pre-RoPE score
    step, H_32 of the codes aside (exact, on the matrix cores): scales with
    the first group butterfly (1.5 per channel), the second group butterfly
    fused with RoPE (4 per channel pair), log2(gh) head butterflies per
    channel, one FMA per channel and query head, and the angle turn of the
    64 pairs (4 each) shared by the gh heads."""
    return 192 + 256 + 128 * (gh.bit_length() - 1) + 128 * g + 256 // gh


ARITHMETIC_BBIT_GQA = {"write": ARITHMETIC_WRITE.replace("2-bit", "b-bit"),
                       "scores": "fp8 digits of a 19-bit fixed-point query x fp4 codes (4-bit codes as two 2-bit "
                                 "planes) on the matrix cores (exact at 1- and 2-bit keys), f32 scale/zero terms",
                       "values": "f16 weights x f16 (plane*s - 1.5 s) on the matrix cores, f32 accumulation",
                       "combine": "f32 merge and un-rotation, output in the query dtype"}


def arithmetic_bbit_g1(vbits):
    """The one-query-head b-bit decode: matrix-core scores at every width, the
    matrix-core value step at 1- and 2-bit values, fp32 FMAs at 4-bit values."""
    return {"write": ARITHMETIC_WRITE.replace("2-bit", "b-bit"),
            "scores": "fp8 digits of a 19-bit fixed-point query (one per row block) x fp4 codes (4-bit codes as "
                      "two 2-bit planes) on the matrix cores, f32 scale/zero terms",
            "values": ("f32 FMA per code, f32 accumulation" if vbits == 4 else
                       "f16 weights fp16(p*s) per value group x f16 codes on the matrix cores, f32 accumulation"),
            "combine": "f32 merge and un-rotation, output in the query dtype"}

PREROLL_MS = 30.0        # untimed calls before each timed phase
FLUSH_BYTES = 1 << 30    # read between timed calls


def file_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(kernel, workload, src_file):
    """HBM bytes per launch from a committed counter summary, or None when
    no summary exists or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != file_sha(src_file):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration():
    import torch
    n = 1 << 28                                # fp32 elements: 1 GiB each way
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty(n, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(a, out=b)                    # one elementwise kernel: read 1 GiB, write 1 GiB
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": 4 * n, "launches": 5}), flush=True)


def copy_bandwidth():
    """Bandwidth of a plain streaming elementwise kernel on this GPU (read
    1 GiB + write 1 GiB per launch): the practical ceiling for context."""
    import torch
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        torch.neg(a, out=b)
    e1.record()
    torch.cuda.synchronize()
    return round(8 * n / (e0.elapsed_time(e1) / 10) / 1e6, 1)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return

    import int2_rotated_kv_amd as kvq
    import workloads as W

    kvq.load_library()
    cfg = W.config(args.config)
    dev = "cuda"
    B, T, H, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    rot = cfg.rot
    workload = cfg.name
    if args.perm:
        if rot != "hadamard":
            sys.exit("--perm applies to the Hadamard workloads (--config 3 or 5)")
        rot, workload = "perm", cfg.name + "_perm"
    if args.varlen:
        workload += "_varlen"
    kbits, vbits = args.kbits, args.vbits
    if (kbits, vbits) != (2, 2):
        workload += f"_k{kbits}v{vbits}"
    GHP = args.prerope
    if GHP:
        if rot != "hadamard" or args.varlen or args.paged or (args.kbits, args.vbits) != (2, 2):
            sys.exit("--prerope applies to the Hadamard workloads (--config 3 or 5), 2-bit, contiguous")
        workload += f"_prerope{GHP}"
    P = args.paged
    if P:
        if P % 64 or rot == "dense":
            sys.exit("--paged P needs P a multiple of 64 and a Hadamard workload")
        workload += f"_paged{P}"
    print(f"[bench] generating {workload} on the GPU", file=sys.stderr, flush=True)
    t0 = time.time()
    K = W.kv_tokens(cfg, "K", device=dev)
    V = W.kv_tokens(cfg, "V", device=dev)
    q = W.queries(cfg, device=dev)
    R = None
    if rot == "dense":
        R = torch.as_tensor(W.dense_rotations(cfg), device=dev).contiguous()
    elif rot == "perm":
        R = torch.as_tensor(W.channel_orders(cfg), dtype=torch.int32, device=dev).contiguous()
    tb, te = cfg.int2_range                    # INT2 tokens of the cache
    if P:
        # every sequence's pages drawn from one shuffled pool (seeded)
        per = (T + P - 1) // P
        pool = np.random.default_rng(np.random.SeedSequence([2000 + cfg.cid, P])).permutation(B * per)
        table = torch.from_numpy(pool.reshape(B, per).astype(np.int32)).to(dev)
        ck = kvq.PagedCache.empty(B * per, H, P, device=dev, bits=kbits)
        cv = kvq.PagedCache.empty(B * per, H, P, device=dev, bits=vbits)
    else:
        ck = kvq.Int2Cache.empty(B, H, T, device=dev, bits=kbits)
        cv = kvq.Int2Cache.empty(B, H, T, device=dev, bits=vbits)

    def write(Kx, Vx, first=None, offsets=None):
        """Rows of every sequence from token `first`, or from offsets[b]."""
        if P:
            offs = offsets if offsets is not None else torch.full((B,), first, dtype=torch.int32, device=dev)
            kvq.kvq_quantize_paged(Kx, Vx, ck, cv, offs, table, rot=rot, R=R)
        elif GHP:
            kvq.kvq_quantize_prerope(Kx, Vx, ck, cv, group_heads=GHP, t_offset=first)
        elif offsets is not None:
            kvq.kvq_quantize(Kx, Vx, ck, cv, rot=rot, R=R, t_offsets=offsets)
        else:
            kvq.kvq_quantize(Kx, Vx, ck, cv, rot=rot, R=R, t_offset=first)
    q0, q1 = cfg.quant_range                   # tokens written by the timed quantize call
    fp16 = {}
    if cfg.n_sink or cfg.n_res:                # fp16 segments, [B, Hkv, n, d]
        fp16 = dict(sink_k=K[:, :tb].permute(0, 2, 1, 3).contiguous(),
                    sink_v=V[:, :tb].permute(0, 2, 1, 3).contiguous(),
                    res_k=K[:, te:].permute(0, 2, 1, 3).contiguous(),
                    res_v=V[:, te:].permute(0, 2, 1, 3).contiguous())
    ws_bytes = (kvq.kvq_decode_workspace_bytes_prerope if GHP else kvq.kvq_decode_workspace_bytes)(
        B, cfg.Hq, H, d, te - tb, cfg.n_sink, cfg.n_res)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    Kq, Vq = K[:, q0:q1], V[:, q0:q1]
    if q0 > tb:                                # rest of the INT2 range, written once (untimed)
        write(K[:, tb:q0], V[:, tb:q0], first=tb)
    ends = None
    if P and not args.varlen:                  # the paged decode takes per-sequence ends
        ends_h = np.full(B, te, np.int32)
        ends = torch.from_numpy(ends_h).to(dev)
    if args.varlen:
        # the whole INT2 range is written once (untimed); sequence b then holds
        # INT2 tokens [tb, ends[b]), and a decode step appends one row at its end
        write(K[:, q0:q1], V[:, q0:q1], first=q0)
        rng = np.random.default_rng(np.random.SeedSequence([1000 + cfg.cid, 77]))
        n_full = te - tb
        ends_h = (tb + rng.integers(n_full // 2, n_full + 1, size=B)).astype(np.int32)
        ends = torch.from_numpy(ends_h).to(dev)
        slots = ends - 1                         # the append rewrites each sequence's last row
        Kq, Vq = K[:, tb:tb + 1], V[:, tb:tb + 1]
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()

    def quant():
        if args.varlen:
            write(Kq, Vq, offsets=slots)
        else:
            write(Kq, Vq, first=q0)

    def decode():
        if GHP:
            kvq.kvq_decode_attention_prerope(q, ck, cv, tb, te, group_heads=GHP, out=out, workspace=ws,
                                             **fp16)
        elif P:
            kvq.kvq_decode_attention_paged(q, ck, cv, tb, ends, te, table, rot=rot, R=R, out=out,
                                           workspace=ws, **fp16)
        else:
            kvq.kvq_decode_attention(q, ck, cv, tb, te, rot=rot, R=R, out=out, workspace=ws,
                                     t_ends=ends, **fp16)

    for _ in range(args.warmup):
        quant()
        decode()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    def preroll(fn, min_ms=PREROLL_MS):
        """Untimed calls of one phase for about min_ms of GPU time, so the
        phase is timed in its own steady state: the clock the part holds
        under a kernel takes some milliseconds to settle after a different
        kernel (right after the dense write kernel, decode runs ~15% slower)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        n = int(min_ms / max(e0.elapsed_time(e1), 1e-3)) + 1
        for _ in range(min(n, 1000)):
            fn()
        torch.cuda.synchronize()

    # Between timed calls a 1 GiB read evicts the caches (the 256 MB MALL
    # included), so no call is served by data the previous one left behind.
    # A read: a copy would leave dirty lines whose write-back lands in the
    # next call (measured ~12% on the decode).
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")

    def flush():
        torch.sum(flush_buf, dim=0, out=flush_out)

    def phase(fn, n):
        preroll(fn)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            flush()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return evs

    torch.cuda.synchronize()
    q_evs = phase(quant, args.steps)
    d_evs = phase(decode, args.steps)
    quant_ms = np.array([a.elapsed_time(b) for a, b in q_evs])
    dec_ms = np.array([a.elapsed_time(b) for a, b in d_evs])
    ms_per_step = float(quant_ms.sum() + dec_ms.sum()) / args.steps   # the timed calls, flushes excluded

    n_q = 1 if args.varlen else q1 - q0
    n_f16 = cfg.n_sink + cfg.n_res
    # INT2 (token, head) units the decode reads: every sequence's own range
    int2_tokens = int((ends_h - tb).sum()) if args.varlen else B * (te - tb)
    r_bytes = {"dense": H * d * d * 4, "perm": H * d * 4}.get(rot, 0)   # R / channel orders, read once
    q_unit = 2 * 256 + row_bytes(kbits) + row_bytes(vbits)
    d_unit = row_bytes(kbits) + row_bytes(vbits)
    assert (kbits, vbits) != (2, 2) or (q_unit, d_unit) == (QUANT_BYTES_PER_TOKEN_HEAD,
                                                             DECODE_BYTES_PER_TOKEN_HEAD)
    q_bytes = B * n_q * H * q_unit + r_bytes
    d_bytes = (int2_tokens * H * d_unit + B * n_f16 * H * FP16_BYTES_PER_TOKEN_HEAD
               + 2 * B * cfg.Hq * d * 2 + r_bytes)
    # mean call time over the timed calls (whole-phase throughput)
    q_ms, d_ms = float(np.mean(quant_ms)), float(np.mean(dec_ms))
    dec_gbs = d_bytes / (d_ms * 1e-3) / 1e9
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9
    q_tok_s = B * n_q / (q_ms * 1e-3)

    csrc = os.path.join(ROOT, "int2_rotated_kv_amd", "csrc")
    q_kernel, q_src = {"dense": ("kv_rotate_quant_dense", "kv_rotate_quant_dense.hip"),
                       "perm": ("kv_rotate_quant_fwht_perm_f16", "kv_rotate_quant.hip")}.get(
                           rot, ("kv_rotate_quant_fwht_f16", "kv_rotate_quant.hip"))
    if (kbits, vbits) != (2, 2) and rot != "dense":
        stem = "kv_rotate_quant_fwht_perm" if rot == "perm" else "kv_rotate_quant_fwht"
        names = [f"{stem}_f16" if b == 2 else f"{stem}_b{b}_f16" for b in (kbits, vbits)]
        q_kernel = names[0] if kbits == vbits else " + ".join(names)
    q_traffic_key = q_kernel
    if GHP:
        # grouped keys and per-head values: two write launches, one traffic record
        q_kernel = (f"kv_rotate_quant_fwht_grouped_f16<{GHP}> + kv_rotate_quant_fwht_f16" if GHP > 1
                    else "kv_rotate_quant_fwht_f16")
        q_traffic_key = "kv_rotate_quant_prerope"
    roof_q = {"bound": "hbm", "achieved": round(q_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
              "frac": round(q_gbs / PEAK_HBM_GBS, 4),
              "traffic": traffic_from_profile(q_traffic_key, workload, os.path.join(csrc, q_src)),
              "kernel": q_kernel, "algorithmic_bytes_per_launch": q_bytes,
              "bytes_per_unit": q_unit, "unit_of_work": "(token, kv head)",
              "units_per_launch": B * n_q * H, "avg_ms": round(q_ms, 4)}
    d_kernel, d_src = (("kv_int2_decode_attn", "kv_decode.hip") if cfg.G == 1
                       else ("kv_int2_decode_attn_gqa", "kv_decode_gqa.hip"))
    if GHP:
        d_kernel, d_src = f"kv_prerope_scores<{GHP}> + kv_int2_decode_attn<4, true>", "kv_decode_prerope.hip"
    # the query preparation is its own launch only for a dense rotation or
    # grouped-query attention; otherwise the attention waves do it
    prep_kernel = (cfg.G > 1 or rot in ("dense", "perm")) and not GHP
    if (kbits, vbits) != (2, 2) and cfg.G == 1:    # the b-bit kernel prepares its query itself
        d_kernel, d_src = f"kv_quant_decode_attn<{kbits},{vbits}>", "kv_decode_generic.hip"
        prep_kernel = rot == "dense"                 # except a dense R's
    elif (kbits, vbits) != (2, 2):                 # grouped-query b-bit kernel, prepared query
        d_kernel, d_src = f"kv_quant_decode_attn_gqa<{kbits},{vbits}>", "kv_decode_gqa_bits.hip"
    # the merge runs one wave per head for one INT2 range, no fp16 tokens and
    # no dense rotation, a block per head otherwise
    merge_kernel = ("kv_combine_wave" if not args.varlen and not P and not fp16 and rot != "dense"
                    else "kv_combine_unrotate")
    roof_d = {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
              "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
              "traffic": traffic_from_profile(d_kernel, workload, os.path.join(csrc, d_src)),
              "kernel": f"decode call ({'kv_prep_query + ' if prep_kernel else ''}{d_kernel} + {merge_kernel})",
              "algorithmic_bytes_per_launch": d_bytes,
              "bytes_per_unit": d_unit, "unit_of_work": "(INT2 token, kv head)",
              "units_per_launch": int2_tokens * H, "avg_ms": round(d_ms, 4)}
    if GHP:
        # the decode call is bound by the score step's vector arithmetic
        ops = int2_tokens * H * prerope_ops_per_unit(GHP, cfg.G)
        tops = ops / (d_ms * 1e-3) / 1e12
        roof_d = {"bound": "alu", "achieved": round(tops, 2), "peak": round(PEAK_VALU_TOPS, 2),
                  "unit": "Top/s", "frac": round(tops / PEAK_VALU_TOPS, 4), "traffic": None,
                  "kernel": f"decode call (kv_rope_table + kv_prerope_scores<{GHP}> + kv_int2_decode_attn<4, true>"
                            f" + {merge_kernel})",
                  "algorithmic_ops_per_launch": ops, "ops_per_unit": prerope_ops_per_unit(GHP, cfg.G),
                  "unit_of_work": "(INT2 token, kv head)", "units_per_launch": int2_tokens * H,
                  "avg_ms": round(d_ms, 4), "hbm_gbs": round(dec_gbs, 1)}
    dominant, other = (roof_q, roof_d) if q_ms >= d_ms else (roof_d, roof_q)
    cache_tag = "int2" if (kbits, vbits) == (2, 2) else f"k{kbits}v{vbits}-bit"

    rec = {
        "metric": METRIC, "value": round(dec_gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"f16 in / {cache_tag} cache", "data": "synthetic",
        "arithmetic": (ARITHMETIC_PREROPE if GHP else
                       (arithmetic_bbit_g1(vbits) if cfg.G == 1 else ARITHMETIC_BBIT_GQA) if (kbits, vbits) != (2, 2) else
                       ARITHMETIC_G1 if cfg.G == 1 else ARITHMETIC_GQA),
        "config": {"workload": workload, "B": B, "T": T, "Hkv": H, "Hq": cfg.Hq, "d": d,
                   "kv_input": "f16",
                   "cache": ("int2 codes + f16 scale/zero, group 32" if (kbits, vbits) == (2, 2) else
                             f"{kbits}-bit key / {vbits}-bit value codes + f16 scale/zero, group 32"),
                   "rotation": rot if not GHP else f"keys: pre-RoPE Hadamard over {GHP} heads; values: Hadamard",
                   "int2_tokens": [tb, te],
                   "quantize_tokens": ("one appended row per sequence, at its own end" if args.varlen
                                       else [q0, q1]),
                   "fp16_tokens": n_f16,
                   **({"int2_ends": {"min": int(ends_h.min()), "max": int(ends_h.max()),
                                     "mean": round(float(ends_h.mean()), 1)}} if args.varlen else {}),
                   **({"page_tokens": P, "pages": int(ck.n_pages)} if P else {})},
        "decode_pct_of_peak": round(100 * dec_gbs / PEAK_HBM_GBS, 2),
        "decode_ms": round(d_ms, 4), "quantize_ms": round(q_ms, 4),
        "quantize_tokens_per_s": round(q_tok_s, 1),
        "quantize_gbs": round(q_gbs, 1),
        "roofline": dominant, "roofline_other": other,
        "timing": {"quantize_ms_median": round(float(np.median(quant_ms)), 4),
                   "decode_ms_median": round(float(np.median(dec_ms)), 4),
                   "quantize_ms_p10_p90": [round(float(np.percentile(quant_ms, 10)), 4),
                                           round(float(np.percentile(quant_ms, 90)), 4)],
                   "decode_ms_p10_p90": [round(float(np.percentile(dec_ms, 10)), 4),
                                         round(float(np.percentile(dec_ms, 90)), 4)]},
    }
    rec["copy_reference_gbs"] = copy_bandwidth()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, rot, K, V, q, R, fp16, kbits, vbits, GHP)
    default_run = (args.config == 3 and not (args.perm or args.varlen or args.paged or GHP)
                   and (kbits, vbits) == (2, 2))
    if default_run and not args.headline_only:
        rec["other_workloads"] = other_workloads(args)
    print(json.dumps(rec), flush=True)


def other_workloads(args):
    """The GQA (dense R, 131072 context) and LLaMA-2-13B (sinks + residual)
    workloads, each measured by a child run of this script, summarized next
    to the headline so that every workload's distance to the roofline is in
    the one line."""
    import subprocess
    out = {}
    for c in (4, 5):
        cmd = [sys.executable, os.path.abspath(__file__), "--config", str(c), "--no-cpu-baseline",
               "--steps", str(args.steps), "--warmup", str(args.warmup)]
        print(f"[bench] child run: config {c}", file=sys.stderr, flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        lines = [ln for ln in res.stdout.splitlines() if ln.startswith("{")]
        if res.returncode != 0 or not lines:
            out[f"config{c}"] = {"error": f"child run failed ({res.returncode})"}
            continue
        r = json.loads(lines[-1])
        out[r["config"]["workload"]] = {
            "decode_ms": r["decode_ms"], "decode_gbs": r["value"], "decode_pct_of_peak": r["decode_pct_of_peak"],
            "quantize_ms": r["quantize_ms"], "quantize_gbs": r["quantize_gbs"],
            "quantize_pct_of_peak": round(100 * r["quantize_gbs"] / PEAK_HBM_GBS, 2),
            "roofline": {k: r["roofline"][k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac")},
            "roofline_other": {k: r["roofline_other"][k] for k in ("kernel", "bound", "achieved", "peak", "unit",
                                                                    "frac")}}
    return out


def cpu_baseline(cfg, rot, K, V, q, R, fp16, kbits=2, vbits=2, ghp=0):
    """The oracle, untouched, on a bounded sample of the same workload:
    batch 0, all KV heads, all tokens of the INT2 range (1/B of the job).
    The sample's inputs are the generator's values (copied from the
    device)."""
    import numpy as np
    from oracle import kvq_oracle as O
    from threadpoolctl import threadpool_info

    tb, te = cfg.int2_range
    if rot == "dense":
        Rm = R.cpu().numpy()
    elif rot == "perm":
        Rm = O.permuted_hadamard_rotation(R.cpu().numpy())
    else:
        Rm = O.hadamard_rotation(cfg.d)
    kh = K[0:1, tb:te].permute(0, 2, 1, 3).contiguous().cpu().numpy()
    vh = V[0:1, tb:te].permute(0, 2, 1, 3).contiguous().cpu().numpy()
    qs = q[0:1].cpu().numpy()
    kw = {k: v[0:1].cpu().numpy() for k, v in fp16.items()}
    t0 = time.perf_counter()
    if ghp:
        # positions are the cache slots [tb, te): the sample's rows shifted to 0
        # would change the angles, so the decode runs on a cache of te slots
        kc = O.quantize_cache_grouped(kh, ghp)
        vc = O.quantize_cache(vh, Rm)
    else:
        kc = O.quantize_cache(kh, Rm, bits=kbits)
        vc = O.quantize_cache(vh, Rm, bits=vbits)
    t1 = time.perf_counter()
    if ghp:
        pad = lambda a: np.concatenate([np.zeros(a.shape[:2] + (tb,) + a.shape[3:], a.dtype), a], axis=2)
        O.decode_attention_prerope(qs, tuple(map(pad, kc)), tuple(map(pad, vc)), tb, te, ghp, **kw)
    else:
        O.decode_attention(qs, kc, vc, 0, te - tb, Rm, **kw)
    t2 = time.perf_counter()
    n_f16 = cfg.n_sink + cfg.n_res
    d_bytes = ((te - tb) * cfg.Hkv * (row_bytes(kbits) + row_bytes(vbits))
               + n_f16 * cfg.Hkv * FP16_BYTES_PER_TOKEN_HEAD
               + 2 * cfg.Hq * cfg.d * 2)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(d_bytes / (t2 - t1) / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"batch 0 of {cfg.B} (all {cfg.Hkv} KV heads, {te - tb} INT2 tokens): oracle "
                      "rotate+quantize+pack of K and V, then oracle decode of the "
                      f"{cfg.Hq} queries; value = decode GB/s over the sample's bytes",
            "quantize_tokens_per_s": round((te - tb) / (t1 - t0), 1),
            "quantize_s": round(t1 - t0, 3), "decode_s": round(t2 - t1, 3),
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
