"""The decode entry point that allocates nothing (kvq_decode_attention_noalloc,
for callers that cannot allocate device memory) against kvq_decode_attention
with a workspace: the same kernels and split plan, so the outputs must be
identical, on two calls in a row (the second smaller, reusing the static
scratch the first left behind), for one and for four query heads per KV head.
Sizes beyond the static scratch are rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

import workloads as W
import int2_rotated_kv_amd as kvq
from parity_util import require_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(cid, B, T, Hkv, Hq):
    cfg = W.small_config(W.config(cid), B=B, T=T, Hkv=Hkv, Hq=Hq)
    K = W.kv_tokens(cfg, "K").to(DEV)
    V = W.kv_tokens(cfg, "V").to(DEV)
    q = W.queries(cfg).to(DEV)
    rot = "dense" if cid == 4 else "hadamard"
    R = torch.as_tensor(W.dense_rotations(cfg), device=DEV).contiguous() if rot == "dense" else None
    ck, cv = kvq.Int2Cache.empty(B, Hkv, T, device=DEV), kvq.Int2Cache.empty(B, Hkv, T, device=DEV)
    kvq.kvq_quantize(K, V, ck, cv, rot=rot, R=R)
    return q, ck, cv, rot, R


@pytest.mark.parametrize("cid,shapes", [(2, [(1, 4096, 32, 32), (1, 700, 8, 8)]),
                                        (4, [(2, 5000, 4, 16), (1, 333, 2, 8)])])
def test_noalloc_decode_matches_workspace_decode(cid, shapes):
    require_gpu()
    for B, T, Hkv, Hq in shapes:
        q, ck, cv, rot, R = _case(cid, B, T, Hkv, Hq)
        ref = kvq.kvq_decode_attention(q, ck, cv, 1, T, rot=rot, R=R)
        out = torch.full_like(q, float("nan"))
        kvq.kvq_decode_attention_noalloc(q, ck, cv, 1, T, rot=rot, R=R, out=out)
        torch.cuda.synchronize()
        print(f"[noalloc] cid={cid} B={B} T={T} Hkv={Hkv} Hq={Hq} "
              f"max|diff|={float((out.float() - ref.float()).abs().max()):.3g}", flush=True)
        assert torch.equal(out, ref)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    require_gpu()
    B, Hkv, Hq, T = 64, 8, 256, 64                       # B*Hq*1 KiB of prepared queries: 16 MiB alone
    q = torch.zeros(B, Hq, 128, dtype=torch.float16, device=DEV)
    ck, cv = kvq.Int2Cache.empty(B, Hkv, T, device=DEV), kvq.Int2Cache.empty(B, Hkv, T, device=DEV)
    need = kvq.kvq_decode_workspace_bytes(B, Hq, Hkv, 128, T)
    assert need > 16 << 20
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attention_noalloc(q, ck, cv, 0, T, rot="hadamard")
    assert e.value.status == 3                           # KVQ_ERR_WORKSPACE_TOO_SMALL
