"""Helpers for the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded inputs, and compare."""
import numpy as np
import torch

from oracle import kvq_oracle as O
import int2_rotated_kv_amd as kvq

SENTINEL = 0xA5


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X: torch.cuda.is_available() is False")
    kvq.load_library()


def empty_cache(B, H, T_cap, device="cuda", bits=2):
    c = kvq.Int2Cache.empty(B, H, T_cap, device=device, bits=bits)
    c.codes.fill_(SENTINEL)
    c.scales.view(torch.uint8).fill_(SENTINEL)
    c.zeros.view(torch.uint8).fill_(SENTINEL)
    return c


def cache_to_numpy(c):
    return (c.codes.cpu().numpy(), c.scales.cpu().numpy(), c.zeros.cpu().numpy())


def cache_from_numpy(packed, scales, zeros, device="cuda"):
    return kvq.Int2Cache(torch.from_numpy(np.ascontiguousarray(packed)).to(device),
                         torch.from_numpy(np.ascontiguousarray(scales)).to(device),
                         torch.from_numpy(np.ascontiguousarray(zeros)).to(device))


def rot_matrix(rot, R=None):
    if rot == "none":
        return None
    if rot == "hadamard":
        return O.hadamard_rotation(128)
    if rot == "perm":
        return O.permuted_hadamard_rotation(R)
    return np.asarray(R, dtype=np.float32)


def compare_codes_at_ties(x_rows, R, gpu, ora, tau=1e-4, max_frac=1e-5, bits=2, tau_sz=1e-5):
    """Rotated-path code check.  x_rows: [..., d] inputs (numpy), gpu/ora:
    (packed, scales, zeros) with matching leading shapes, codes `bits` wide.
    Returns stats.

    Every differing code must differ by one and sit at a rounding tie of the
    exact quantizer argument (within tau of k + 1/2), unless its group's
    scale or zero differs by one fp16 ulp between the two sides.  A scale
    or zero may differ only by one fp16 ulp, and only where the exact value
    (fp64 rotation: (max - min)/L, or min) lies within tau_sz * max|row| of
    the rounding boundary between the two fp16 values, i.e. where rounding
    of the rotation can decide it.
    """
    gp, gs, gz = gpu
    op, os_, oz = ora
    gc = O.unpack_codes(gp, bits).astype(np.int16)
    oc = O.unpack_codes(op, bits).astype(np.int16)
    diff = gc != oc
    n = gc.size
    s_diff = gs.view(np.uint16) != os_.view(np.uint16)
    z_diff = gz.view(np.uint16) != oz.view(np.uint16)
    sz_diff = s_diff | z_diff
    for g_, o_, what in ((gs, os_, "scale"), (gz, oz, "zero")):
        g64, o64 = g_.astype(np.float64), o_.astype(np.float64)
        ulp = np.spacing(np.maximum(np.abs(g_), np.abs(o_)).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(g64 - o64) <= ulp), f"{what} differs by more than one fp16 ulp"
    if sz_diff.any():
        y64 = np.asarray(x_rows, dtype=np.float64)
        if R is not None:
            y64 = y64 @ np.asarray(R, dtype=np.float64)
        d = y64.shape[-1]
        yg = y64.reshape(*y64.shape[:-1], d // 32, 32)
        mn, mx = yg.min(-1), yg.max(-1)
        row = np.abs(y64).max(-1, keepdims=True)
        L = (1 << bits) - 1
        for mask, exact, g_, o_, what in ((s_diff, (mx - mn) / L, gs, os_, "scale"),
                                          (z_diff, mn, gz, oz, "zero")):
            if mask.any():
                mid = (g_.astype(np.float64) + o_.astype(np.float64)) / 2
                off = np.abs(exact - mid)[mask]
                lim = (tau_sz * np.broadcast_to(row, mask.shape))[mask]
                assert np.all(off <= lim), f"{what} differs away from an fp16 rounding boundary"
    stats = dict(elements=n, code_mismatch=int(diff.sum()),
                 group_scale_zero_diff=int(sz_diff.sum()), groups=int(gs.size))
    if diff.any():
        assert np.all(np.abs(gc - oc)[diff] == 1), "code differs by more than one"
        dist = O.tie_distance(x_rows, R, os_, oz)
        grp_flag = np.repeat(sz_diff, 32, axis=-1)
        ok = (dist <= tau) | grp_flag
        bad = diff & ~ok
        assert not bad.any(), f"{int(bad.sum())} code mismatches away from ties"
        assert diff.sum() / n <= max_frac, f"mismatch fraction {diff.sum() / n:.3g}"
    return stats


def normwise_rel_err(out, ref):
    """max over rows (b, h) of max_c |out - ref| / max_c |ref|."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(out - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float((num / den).max())


def elementwise_rel_err(out, ref, floor=1e-3):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.maximum(np.abs(ref), floor * np.abs(ref).max(axis=-1, keepdims=True))
    return float((np.abs(out - ref) / den).max())
