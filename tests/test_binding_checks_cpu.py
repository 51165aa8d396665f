"""The Python binding rejects malformed tensors before the C ABI is reached.

The library takes raw device pointers and trusts the sizes its shape
arguments imply, so a cache with a smaller batch, a sliced cache view, a
host tensor or a rotation of the wrong shape would otherwise become an
out-of-bounds device access.  Each case below must raise ValueError without
loading or calling the library (load_library is replaced by a function that
fails the test).  CPU only: the shape checks run before the device check.
"""
import pytest
import torch

import int2_rotated_kv_amd as kvq
from int2_rotated_kv_amd import kvq as K


@pytest.fixture(autouse=True)
def _no_library(monkeypatch):
    def _fail():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(K, "load_library", _fail)


def _rows(B=2, T=8, H=4, dtype=torch.float16):
    return torch.zeros(B, T, H, 128, dtype=dtype)


def _cache(B=2, H=4, T=64, bits=2):
    return kvq.Int2Cache.empty(B, H, T, device="cpu", bits=bits)


def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_quantize_host_tensors_rejected():
    _raises(lambda: kvq.kvq_quantize(_rows(), None, _cache(), None), "GPU")


def test_quantize_cache_batch_mismatch():
    _raises(lambda: kvq.kvq_quantize(_rows(B=2), None, _cache(B=1), None), "leading dims")


def test_quantize_cache_head_mismatch():
    _raises(lambda: kvq.kvq_quantize(_rows(H=4), None, _cache(H=2), None), "leading dims")


def test_quantize_sliced_cache_view():
    c = _cache(T=64)
    view = kvq.Int2Cache(c.codes[:, :, :32], c.scales[:, :, :32], c.zeros[:, :, :32])
    _raises(lambda: kvq.kvq_quantize(_rows(), None, view, None), "contiguous")


def test_quantize_wrong_cache_dtype():
    c = _cache()
    bad = kvq.Int2Cache(c.codes, c.scales.float().half().view(torch.int16), c.zeros)
    _raises(lambda: kvq.kvq_quantize(_rows(), None, bad, None), "4-D")


def test_quantize_rows_without_cache():
    _raises(lambda: kvq.kvq_quantize(_rows(), _rows(), _cache(), None), "neither")


def test_quantize_bad_channel_stride():
    x = torch.zeros(2, 8, 4, 256, dtype=torch.float16)[..., ::2]
    _raises(lambda: kvq.kvq_quantize(x, None, _cache(), None), "unit channel stride")


@pytest.mark.parametrize("rot,R,match", [
    ("dense", None, "dense"),
    ("dense", torch.zeros(4, 128, 128, dtype=torch.float16), "dense"),
    ("dense", torch.zeros(3, 128, 128), "dense"),
    ("perm", torch.zeros(4, 128, dtype=torch.int64), "perm"),
    ("perm", torch.zeros(4, 64, dtype=torch.int32), "perm"),
    ("hadamard", torch.zeros(4, 128, 128), "takes no R"),
    ("rotate", None, "unknown rotation"),
])
def test_quantize_bad_rotation(rot, R, match):
    _raises(lambda: kvq.kvq_quantize(_rows(), None, _cache(), None, rot=rot, R=R), match)


def test_quantize_bad_offsets():
    _raises(lambda: kvq.kvq_quantize(_rows(), None, _cache(), None,
                                     t_offsets=torch.zeros(2, dtype=torch.int64)), "t_offsets")
    _raises(lambda: kvq.kvq_quantize(_rows(), None, _cache(), None,
                                     t_offsets=torch.zeros(3, dtype=torch.int32)), "t_offsets")


def _q(B=2, Hq=8, dtype=torch.float16):
    return torch.zeros(B, Hq, 128, dtype=dtype)


def test_decode_host_tensors_rejected():
    _raises(lambda: kvq.kvq_decode_attention(_q(), _cache(), _cache(), 0, 64), "GPU")


def test_decode_cache_batch_mismatch():
    _raises(lambda: kvq.kvq_decode_attention(_q(B=2), _cache(B=1), _cache(B=1), 0, 64), "leading dims")


def test_decode_range_past_cache():
    _raises(lambda: kvq.kvq_decode_attention(_q(), _cache(T=64), _cache(T=64), 0, 65), "outside")


def test_decode_query_not_contiguous():
    q = torch.zeros(2, 128, 8, dtype=torch.float16).transpose(1, 2)
    _raises(lambda: kvq.kvq_decode_attention(q, _cache(), _cache(), 0, 64), "contiguous")


def test_decode_heads_not_multiple():
    _raises(lambda: kvq.kvq_decode_attention(_q(Hq=6), _cache(H=4), _cache(H=4), 0, 64), "multiple")


def test_decode_sink_shape():
    sk = torch.zeros(2, 3, 4, 128, dtype=torch.float16)
    _raises(lambda: kvq.kvq_decode_attention(_q(), _cache(), _cache(), 0, 64, sink_k=sk, sink_v=sk),
            "sink")
    sk = torch.zeros(2, 4, 4, 128, dtype=torch.float32)
    _raises(lambda: kvq.kvq_decode_attention(_q(), _cache(), _cache(), 0, 64, sink_k=sk, sink_v=sk),
            "sink")
    sk = torch.zeros(2, 4, 4, 128, dtype=torch.float16)
    _raises(lambda: kvq.kvq_decode_attention(_q(), _cache(), _cache(), 0, 64, sink_k=sk), "sink")


def test_decode_out_shape():
    _raises(lambda: kvq.kvq_decode_attention(_q(), _cache(), _cache(), 0, 64,
                                             out=torch.zeros(2, 8, 64, dtype=torch.float16)), "out")


def test_decode_bad_ends():
    _raises(lambda: kvq.kvq_decode_attention(_q(), _cache(), _cache(), 0, 64,
                                             t_ends=torch.zeros(2, dtype=torch.int64)), "t_ends")


def test_decode_mixed_sides():
    _raises(lambda: kvq.kvq_decode_attention(_q(), _cache(), None, 0, 64), "both cache sides")


def _paged(n=6, H=4, P=64, bits=2):
    return kvq.PagedCache.empty(n, H, P, device="cpu", bits=bits)


def test_paged_quantize_bad_table():
    offs = torch.zeros(2, dtype=torch.int32)
    _raises(lambda: kvq.kvq_quantize_paged(_rows(), None, _paged(), None, offs,
                                           torch.zeros(2, 3, dtype=torch.int64)), "block_table")
    _raises(lambda: kvq.kvq_quantize_paged(_rows(), None, _paged(), None, offs,
                                           torch.zeros(3, 3, dtype=torch.int32)), "block_table")


def test_paged_quantize_head_mismatch():
    offs = torch.zeros(2, dtype=torch.int32)
    table = torch.zeros(2, 3, dtype=torch.int32)
    _raises(lambda: kvq.kvq_quantize_paged(_rows(H=4), None, _paged(H=2), None, offs, table),
            "leading dims")


def test_paged_decode_pool_mismatch_and_capacity():
    ends = torch.zeros(2, dtype=torch.int32)
    table = torch.zeros(2, 3, dtype=torch.int32)
    _raises(lambda: kvq.kvq_decode_attention_paged(_q(), _paged(n=6), _paged(n=5), 0, ends, 64, table),
            "pool")
    _raises(lambda: kvq.kvq_decode_attention_paged(_q(), _paged(), _paged(), 0, ends, 3 * 64 + 1, table),
            "capacity")
    _raises(lambda: kvq.kvq_decode_attention_paged(_q(), _paged(), _paged(), 0, ends, 64, table), "GPU")
