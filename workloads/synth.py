"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds no part of the method (no rotation, quantization or
attention).  It only draws inputs, and both the HIP path and the CPU
oracle are fed from it.

Normal deviates come from a counter-based generator so that any slice of a
large tensor can be regenerated on the CPU (for the oracle) exactly as it
was generated on the GPU:

    h(key, i) = lowbias32( lo32(i) ^ lowbias32( hi32(i) ^ lowbias32(key) ) )
    lowbias32(x): x ^= x >> 16; x *= 0x7feb352d; x ^= x >> 15;
                  x *= 0x846ca68b; x ^= x >> 16          (all mod 2**32)
    u1 = (h(2k, i) + 0.5) / 2**32,   u2 = (h(2k+1, i) + 0.5) / 2**32
    z  = sqrt(-2 ln u1) * cos(2 pi u2)                     (Box-Muller, fp64)

lowbias32 is the 32-bit integer hash published by C. Wellons ("hash
prospector", 2018).  The integer part is exact on every device; the fp64
transcendental step can differ by an ulp between CPU and GPU libraries,
which changes an fp16 (or fp32) input only with probability ~2**-40
(~2**-27) per element.

Small per-head parameters (outlier channels, channel scales, dense
rotations) come from numpy's seeded default_rng and are shared by both
sides as arrays.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

_M32 = 0xFFFFFFFF

# stream ids (second entry of every SeedSequence / counter key)
S_K, S_V, S_Q, S_SIGMA_K, S_SIGMA_V, S_ROT = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    B: int
    T: int          # context length (tokens held per sequence)
    Hkv: int
    Hq: int
    d: int
    dtype: str      # "f16" or "f32": K, V and q element type
    rot: str        # "hadamard" or "dense"
    outliers: str   # "fixed", "random4x15", "loguniform", "none"
    n_sink: int = 0
    n_res: int = 0
    sink_gain: float = 1.0
    t_new: int = 0  # tokens written by the timed quantize call (0 = all)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.float32

    @property
    def int2_range(self):
        """INT2 token range [t_begin, t_end) of the cache."""
        return self.n_sink, self.T - self.n_res

    @property
    def quant_range(self):
        """Token range [t0, t1) written by the timed quantize call."""
        t_begin, t_end = self.int2_range
        if self.t_new:
            return t_end - self.t_new, t_end
        return t_begin, t_end


CONFIGS = {
    # tiny single-head case, fp32, channels 3 and 17 scaled x20
    1: Config(1, "tiny_single_head_T1024", B=1, T=1024, Hkv=1, Hq=1, d=128,
              dtype="f32", rot="hadamard", outliers="fixed"),
    # LLaMA-2-7B-shaped layer, 4 outlier channels per head x15
    2: Config(2, "llama2_7b_layer_T4096", B=1, T=4096, Hkv=32, Hq=32, d=128,
              dtype="f16", rot="hadamard", outliers="random4x15"),
    # throughput case, per-(head, channel) scales log-uniform in [0.5, 20]
    3: Config(3, "throughput_B16_T32768_H32", B=16, T=32768, Hkv=32, Hq=32,
              d=128, dtype="f16", rot="hadamard", outliers="loguniform"),
    # GQA 32q/8kv with a dense per-head orthogonal rotation, prefill 32768
    4: Config(4, "gqa_dense_B4_T131072_Hkv8", B=4, T=131072, Hkv=8, Hq=32,
              d=128, dtype="f16", rot="dense", outliers="none",
              t_new=32768),
    # LLaMA-2-13B-shaped sink / residual mix
    5: Config(5, "llama2_13b_sinks_B8_T65536_H40", B=8, T=65536, Hkv=40,
              Hq=40, d=128, dtype="f16", rot="hadamard",
              outliers="random4x15", n_sink=4, n_res=128, sink_gain=50.0),
}


def config(cid: int) -> Config:
    return CONFIGS[cid]


def small_config(base: Config, **kw) -> Config:
    """A reduced copy of a config (same recipe, smaller shapes)."""
    return dataclasses.replace(base, **kw)


# --------------------------------------------------------------------------
# counter-based normal generator (identical integer path on CPU and GPU)
# --------------------------------------------------------------------------
def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2**32 without int64 overflow (x < 2**32)."""
    lo, hi = c & 0xFFFF, c >> 16
    return ((x * lo) + (((x * hi) & 0xFFFF) << 16)) & _M32


def _lowbias32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _lowbias32_int(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    x ^= x >> 16
    return x


def _hash(key: int, idx: torch.Tensor) -> torch.Tensor:
    hk = _lowbias32_int(key)
    hi = (idx >> 32) & _M32
    lo = idx & _M32
    return _lowbias32(lo ^ _lowbias32(hi ^ hk))


def normal_at(key: int, idx: torch.Tensor) -> torch.Tensor:
    """fp64 standard normal deviates at counter positions idx (int64)."""
    h1 = _hash(2 * key, idx).to(torch.float64)
    h2 = _hash(2 * key + 1, idx).to(torch.float64)
    u1 = (h1 + 0.5) * (1.0 / 4294967296.0)
    u2 = (h2 + 0.5) * (1.0 / 4294967296.0)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def _key(cfg: Config, stream: int) -> int:
    return ((1000 + cfg.cid) * 64 + stream) & _M32


# --------------------------------------------------------------------------
# per-head parameters
# --------------------------------------------------------------------------
def channel_sigma(cfg: Config, which: str) -> np.ndarray:
    """Per-(KV head, channel) standard deviation, float64 [Hkv, d]."""
    stream = S_SIGMA_K if which == "K" else S_SIGMA_V
    rng = np.random.default_rng(np.random.SeedSequence([1000 + cfg.cid, stream]))
    sig = np.ones((cfg.Hkv, cfg.d), np.float64)
    if cfg.outliers == "fixed":
        sig[:, 3] = 20.0
        sig[:, 17] = 20.0
    elif cfg.outliers == "random4x15":
        for h in range(cfg.Hkv):
            ch = rng.choice(cfg.d, size=4, replace=False)
            sig[h, ch] = 15.0
    elif cfg.outliers == "loguniform":
        sig = np.exp(rng.uniform(math.log(0.5), math.log(20.0),
                                 size=(cfg.Hkv, cfg.d)))
    elif cfg.outliers != "none":
        raise ValueError(cfg.outliers)
    return sig


def dense_rotations(cfg: Config) -> np.ndarray:
    """Per-KV-head orthogonal matrices from the QR of a seeded Gaussian.

    R_h = Q diag(sign(diag(Rq))) with Q, Rq = qr(G_h), G_h ~ N(0,1) in
    fp64, then cast to fp32 (the fp32 array is the library input).
    Returns float32 [Hkv, d, d].
    """
    rng = np.random.default_rng(np.random.SeedSequence([1000 + cfg.cid, S_ROT]))
    out = np.empty((cfg.Hkv, cfg.d, cfg.d), np.float32)
    for h in range(cfg.Hkv):
        g = rng.standard_normal((cfg.d, cfg.d))
        qm, rm = np.linalg.qr(g)
        out[h] = (qm * np.sign(np.diag(rm))[None, :]).astype(np.float32)
    return out


def channel_orders(cfg: Config) -> np.ndarray:
    """Per-KV-head channel orders for the reordered Hadamard rotation: the
    channels of each head sorted by their K standard deviation, largest
    first (ties by channel index), i.e. ordered by outlier magnitude.
    Returns int32 [Hkv, d], each row a permutation of 0..d-1."""
    sig = channel_sigma(cfg, "K")
    return np.stack([np.argsort(-sig[h], kind="stable") for h in range(cfg.Hkv)]).astype(np.int32)


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------
def kv_tokens(cfg: Config, which: str, b0: int = 0, b1: int | None = None,
              t0: int = 0, t1: int | None = None, device="cpu",
              out: torch.Tensor | None = None, h0: int = 0,
              h1: int | None = None, chunk_elems: int = 1 << 25) -> torch.Tensor:
    """Token-major K or V rows [b1-b0, t1-t0, h1-h0, d] in the config dtype.

    Element (b, t, h, c) is normal_at(key, ((b*T + t)*Hkv + h)*d + c)
    times sigma[h, c], times the sink gain for t < n_sink, so any slice of
    batches, tokens and heads is reproducible on its own.
    """
    b1 = cfg.B if b1 is None else b1
    t1 = cfg.T if t1 is None else t1
    h1 = cfg.Hkv if h1 is None else h1
    nb, nt, nh = b1 - b0, t1 - t0, h1 - h0
    d = cfg.d
    if out is None:
        out = torch.empty((nb, nt, nh, d), dtype=cfg.torch_dtype, device=device)
    key = _key(cfg, S_K if which == "K" else S_V)
    sig = torch.as_tensor(channel_sigma(cfg, which)[h0:h1], dtype=torch.float64,
                          device=out.device)
    row = cfg.Hkv * d
    ar = ((torch.arange(h0, h1, dtype=torch.int64, device=out.device) * d)[:, None]
          + torch.arange(d, dtype=torch.int64, device=out.device)[None, :]).reshape(-1)
    rows_per_chunk = max(1, chunk_elems // (nh * d))
    for bi in range(nb):
        b = b0 + bi
        for ts in range(0, nt, rows_per_chunk):
            te = min(nt, ts + rows_per_chunk)
            tok = torch.arange(t0 + ts, t0 + te, dtype=torch.int64,
                               device=out.device)
            idx = ((b * cfg.T + tok) * row)[:, None] + ar[None, :]
            z = normal_at(key, idx).view(te - ts, nh, d) * sig[None]
            if cfg.n_sink and cfg.sink_gain != 1.0:
                gain = torch.where(tok < cfg.n_sink, cfg.sink_gain, 1.0)
                z = z * gain.to(torch.float64)[:, None, None]
            out[bi, ts:te] = z.to(out.dtype)
    return out


def queries(cfg: Config, device="cpu") -> torch.Tensor:
    """Decode queries [B, Hq, d], N(0,1), in the config dtype."""
    n = cfg.B * cfg.Hq * cfg.d
    idx = torch.arange(n, dtype=torch.int64, device=device)
    z = normal_at(_key(cfg, S_Q), idx).view(cfg.B, cfg.Hq, cfg.d)
    return z.to(cfg.torch_dtype)


def head_major(x_tok: torch.Tensor) -> torch.Tensor:
    """[B, T, H, d] token-major -> contiguous [B, H, T, d] copy."""
    return x_tok.permute(0, 2, 1, 3).contiguous()
