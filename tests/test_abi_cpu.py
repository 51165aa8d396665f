"""CPU checks of the C-ABI library: it loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call.

No call here reaches a kernel launch: every call fails validation (fake,
never dereferenced pointer values are used only where validation stops
first), except the pure-arithmetic workspace query.
"""
import ctypes
import os
import re
import subprocess

import pytest

from int2_rotated_kv_amd import kvq as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

FAKE = 0x10000          # 16-byte aligned, never dereferenced
FAKE_MISALIGNED = 0x10008


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return K.load_library()


def test_header_declares_the_boundary():
    assert header_functions() == sorted(K.EXPORTED_SYMBOLS)


def test_library_exports_every_header_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", K.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(kvq_\w+)", out))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    hdr = open(os.path.join(ROOT, "include", "kvq.h")).read()
    assert K.kvq_abi_version() == int(re.search(r"#define KVQ_ABI_VERSION (\d+)", hdr).group(1))
    names = [K.kvq_status_str(s) for s in range(5)]
    assert names == ["KVQ_OK", "KVQ_ERR_INVALID_ARG", "KVQ_ERR_UNSUPPORTED",
                     "KVQ_ERR_WORKSPACE_TOO_SMALL", "KVQ_ERR_HIP"]
    assert K.kvq_status_str(99) == "KVQ_ERR_UNKNOWN"


def _cache(T_cap=64, codes=FAKE, scales=FAKE, zeros=FAKE):
    return K.kvq_int2_cache(codes, scales, zeros, T_cap)


def _quant(lib, **kw):
    a = dict(K=FAKE, V=FAKE, dt=K.KVQ_F16, B=1, T=8, H=2, d=128, sb=8 * 2 * 128,
             st=2 * 128, sh=128, rot=K.KVQ_ROT_HADAMARD, R=None, group=32, toff=0,
             kc=_cache(), vc=_cache())
    a.update(kw)
    kc = ctypes.byref(a["kc"]) if a["kc"] is not None else None
    vc = ctypes.byref(a["vc"]) if a["vc"] is not None else None
    return lib.kvq_quantize(a["K"], a["V"], a["dt"], a["B"], a["T"], a["H"], a["d"],
                            a["sb"], a["st"], a["sh"], a["rot"], a["R"], a["group"],
                            a["toff"], kc, vc, None)


QUANT_ERRORS = [
    (dict(d=64), K.KVQ_ERR_UNSUPPORTED),
    (dict(group=64), K.KVQ_ERR_UNSUPPORTED),
    (dict(dt=7), K.KVQ_ERR_INVALID_ARG),
    (dict(rot=9), K.KVQ_ERR_INVALID_ARG),
    (dict(B=-1), K.KVQ_ERR_INVALID_ARG),
    (dict(T=-1), K.KVQ_ERR_INVALID_ARG),
    (dict(H=0), K.KVQ_ERR_INVALID_ARG),
    (dict(toff=-1), K.KVQ_ERR_INVALID_ARG),
    (dict(st=-128), K.KVQ_ERR_INVALID_ARG),
    (dict(K=None), K.KVQ_ERR_INVALID_ARG),                 # input without cache
    (dict(K=None, kc=None, V=None, vc=None), K.KVQ_ERR_INVALID_ARG),
    (dict(K=FAKE_MISALIGNED), K.KVQ_ERR_INVALID_ARG),
    (dict(sh=100), K.KVQ_ERR_INVALID_ARG),                 # row start not 16-byte aligned
    (dict(kc=_cache(codes=0)), K.KVQ_ERR_INVALID_ARG),
    (dict(kc=_cache(scales=FAKE_MISALIGNED)), K.KVQ_ERR_INVALID_ARG),
    (dict(kc=_cache(T_cap=0)), K.KVQ_ERR_INVALID_ARG),
    (dict(toff=60), K.KVQ_ERR_INVALID_ARG),                # 60 + 8 > T_cap 64
    (dict(vc=_cache(T_cap=4)), K.KVQ_ERR_INVALID_ARG),
    (dict(rot=K.KVQ_ROT_HADAMARD, R=FAKE), K.KVQ_ERR_INVALID_ARG),
    (dict(rot=K.KVQ_ROT_DENSE, R=None), K.KVQ_ERR_INVALID_ARG),
    (dict(rot=K.KVQ_ROT_DENSE, R=FAKE, dt=K.KVQ_F32, sb=8 * 2 * 128, st=256, sh=128),
     K.KVQ_ERR_UNSUPPORTED),
    (dict(B=70000), K.KVQ_ERR_UNSUPPORTED),                # grid z limit
    (dict(rot=K.KVQ_ROT_PERM_HADAMARD, R=None), K.KVQ_ERR_INVALID_ARG),
    (dict(rot=K.KVQ_ROT_PERM_HADAMARD, R=FAKE_MISALIGNED), K.KVQ_ERR_INVALID_ARG),
    (dict(rot=K.KVQ_ROT_PERM_HADAMARD, R=FAKE, dt=K.KVQ_F32, sb=8 * 2 * 128, st=256, sh=128),
     K.KVQ_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,want", QUANT_ERRORS, ids=[str(e[0]) for e in QUANT_ERRORS])
def test_quantize_rejects(lib, kw, want):
    assert _quant(lib, **kw) == want


def test_quantize_empty_is_noop(lib):
    # validated, then nothing to do: returns before any HIP call
    assert _quant(lib, T=0) == K.KVQ_OK
    assert _quant(lib, B=0) == K.KVQ_OK


def _decode(lib, **kw):
    a = dict(q=FAKE, qdt=K.KVQ_F16, B=2, Hq=4, Hkv=2, d=128, kc=_cache(), vc=_cache(),
             tb=0, te=64, rot=K.KVQ_ROT_HADAMARD, R=None, group=32, sk=None, sv=None,
             ns=0, rk=None, rv=None, nr=0, scale=0.0, out=FAKE, odt=K.KVQ_F16,
             ws=FAKE * 16, wsb=1 << 30)
    a.update(kw)
    kc = ctypes.byref(a["kc"]) if a["kc"] is not None else None
    vc = ctypes.byref(a["vc"]) if a["vc"] is not None else None
    return lib.kvq_decode_attention(a["q"], a["qdt"], a["B"], a["Hq"], a["Hkv"], a["d"],
                                    kc, vc, a["tb"], a["te"], a["rot"], a["R"], a["group"],
                                    a["sk"], a["sv"], a["ns"], a["rk"], a["rv"], a["nr"],
                                    a["scale"], a["out"], a["odt"], a["ws"], a["wsb"], None)


DECODE_ERRORS = [
    (dict(d=256), K.KVQ_ERR_UNSUPPORTED),
    (dict(group=16), K.KVQ_ERR_UNSUPPORTED),
    (dict(q=None), K.KVQ_ERR_INVALID_ARG),
    (dict(out=FAKE_MISALIGNED), K.KVQ_ERR_INVALID_ARG),
    (dict(qdt=3), K.KVQ_ERR_INVALID_ARG),
    (dict(Hq=3), K.KVQ_ERR_INVALID_ARG),                   # not a multiple of Hkv
    (dict(B=0), K.KVQ_ERR_INVALID_ARG),
    (dict(tb=10, te=5), K.KVQ_ERR_INVALID_ARG),
    (dict(te=65), K.KVQ_ERR_INVALID_ARG),                  # beyond T_cap
    (dict(kc=None), K.KVQ_ERR_INVALID_ARG),
    (dict(vc=_cache(zeros=0)), K.KVQ_ERR_INVALID_ARG),
    (dict(ns=4), K.KVQ_ERR_INVALID_ARG),                   # sinks without pointers
    (dict(nr=2, rk=FAKE, rv=None), K.KVQ_ERR_INVALID_ARG),
    (dict(nr=9000, rk=FAKE, rv=FAKE), K.KVQ_ERR_UNSUPPORTED),
    (dict(tb=0, te=0), K.KVQ_ERR_INVALID_ARG),             # no tokens at all
    (dict(rot=K.KVQ_ROT_DENSE), K.KVQ_ERR_INVALID_ARG),    # dense without R
    (dict(rot=K.KVQ_ROT_PERM_HADAMARD), K.KVQ_ERR_INVALID_ARG),   # permutation missing
    (dict(rot=K.KVQ_ROT_NONE, R=FAKE), K.KVQ_ERR_INVALID_ARG),
    (dict(ws=None), K.KVQ_ERR_INVALID_ARG),
    (dict(ws=FAKE + 16), K.KVQ_ERR_INVALID_ARG),           # workspace not 256-aligned
    (dict(wsb=100), K.KVQ_ERR_WORKSPACE_TOO_SMALL),
    (dict(scale=float("nan")), K.KVQ_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,want", DECODE_ERRORS, ids=[str(e[0]) for e in DECODE_ERRORS])
def test_decode_rejects(lib, kw, want):
    assert _decode(lib, **kw) == want


def test_quantize_at_rejects(lib):
    a = dict(K=FAKE, V=FAKE, dt=K.KVQ_F16, B=1, T=8, H=2, d=128, sb=8 * 2 * 128,
             st=2 * 128, sh=128, rot=K.KVQ_ROT_HADAMARD, R=None, group=32)
    kc, vc = _cache(), _cache()

    def call(offs, T=8, kcache=kc):
        return lib.kvq_quantize_at(a["K"], a["V"], a["dt"], a["B"], T, a["H"], a["d"], a["sb"],
                                   a["st"], a["sh"], a["rot"], a["R"], a["group"], offs,
                                   ctypes.byref(kcache), ctypes.byref(vc), None)
    assert call(None) == K.KVQ_ERR_INVALID_ARG                 # offsets missing
    assert call(FAKE + 2) == K.KVQ_ERR_INVALID_ARG             # not 4-byte aligned
    assert call(FAKE, T=65) == K.KVQ_ERR_INVALID_ARG           # T_new > T_cap
    assert call(FAKE, T=0) == K.KVQ_OK                         # nothing to write


def test_decode_varlen_rejects(lib):
    def call(t_ends, te_max=64, **kw):
        a = dict(q=FAKE, qdt=K.KVQ_F16, B=2, Hq=4, Hkv=2, d=128, kc=_cache(), vc=_cache(),
                 tb=0, rot=K.KVQ_ROT_HADAMARD, R=None, group=32, out=FAKE, odt=K.KVQ_F16,
                 ws=FAKE * 16, wsb=1 << 30)
        a.update(kw)
        return lib.kvq_decode_attention_varlen(
            a["q"], a["qdt"], a["B"], a["Hq"], a["Hkv"], a["d"], ctypes.byref(a["kc"]),
            ctypes.byref(a["vc"]), a["tb"], t_ends, te_max, a["rot"], a["R"], a["group"],
            None, None, 0, None, None, 0, 0.0, a["out"], a["odt"], a["ws"], a["wsb"], None)
    assert call(None) == K.KVQ_ERR_INVALID_ARG                 # ends missing
    assert call(FAKE + 2) == K.KVQ_ERR_INVALID_ARG             # not 4-byte aligned
    assert call(FAKE, te_max=65) == K.KVQ_ERR_INVALID_ARG      # bound beyond T_cap
    assert call(FAKE, wsb=100) == K.KVQ_ERR_WORKSPACE_TOO_SMALL


def test_workspace_bytes():
    # invalid sizes give 0
    assert K.kvq_decode_workspace_bytes(0, 4, 2, 128, 10) == 0
    assert K.kvq_decode_workspace_bytes(1, 3, 2, 128, 10) == 0
    assert K.kvq_decode_workspace_bytes(1, 4, 2, 64, 10) == 0
    # query block (1 KiB per head, 256-aligned) + 132 floats per (head, split)
    qprep = 16 * 32 * 1024
    ws = K.kvq_decode_workspace_bytes(16, 32, 32, 128, 32768)
    assert ws > qprep and (ws - qprep) % (16 * 32 * 132 * 4) == 0
    n_splits = (ws - qprep) // (16 * 32 * 132 * 4)
    assert 1 <= n_splits <= 32768 // 256
    # no INT2 tokens: only the query block
    assert K.kvq_decode_workspace_bytes(1, 4, 2, 128, 0, 4, 8) == 4 * 1024
    # more tokens never need fewer splits
    prev = 0
    for n in (1, 100, 1000, 10000, 100000, 1000000):
        w = K.kvq_decode_workspace_bytes(1, 8, 8, 128, n)
        assert w >= prev
        prev = w


def _qcache(bits, T_cap=64):
    return K.kvq_quant_cache(FAKE, FAKE, FAKE, T_cap, bits)


def test_quantize_bits_rejects(lib):
    """Code widths: 1, 2 or 4 bits per side; 1 and 4 need fp16 rows with
    the (reordered) Hadamard rotation."""
    def call(kb, vb, dt=K.KVQ_F16, rot=K.KVQ_ROT_HADAMARD, R=None):
        return lib.kvq_quantize_bits(FAKE, FAKE, dt, 1, 8, 2, 128, 8 * 2 * 128, 2 * 128, 128,
                                     rot, R, 32, 0, ctypes.byref(_qcache(kb)),
                                     ctypes.byref(_qcache(vb)), None)
    assert call(3, 2) == K.KVQ_ERR_INVALID_ARG                  # no 3-bit codes
    assert call(2, 8) == K.KVQ_ERR_INVALID_ARG
    assert call(4, 2, dt=K.KVQ_F32) == K.KVQ_ERR_UNSUPPORTED    # fp32 rows at 4 bits
    assert call(2, 1, rot=K.KVQ_ROT_NONE) == K.KVQ_ERR_UNSUPPORTED
    assert call(4, 4, dt=K.KVQ_F32, rot=K.KVQ_ROT_DENSE, R=FAKE) == K.KVQ_ERR_UNSUPPORTED
    assert call(4, 4, rot=K.KVQ_ROT_DENSE, R=None) == K.KVQ_ERR_INVALID_ARG   # dense needs R
    assert call(4, 2, rot=K.KVQ_ROT_PERM_HADAMARD) == K.KVQ_ERR_INVALID_ARG   # no channel order


def test_decode_bits_rejects(lib):
    def call(kb, vb, rot=K.KVQ_ROT_HADAMARD, R=None, wsb=1 << 30):
        return lib.kvq_decode_attention_bits(
            FAKE, K.KVQ_F16, 2, 4, 2, 128, ctypes.byref(_qcache(kb)), ctypes.byref(_qcache(vb)),
            0, 64, rot, R, 32, None, None, 0, None, None, 0, 0.0, FAKE, K.KVQ_F16,
            FAKE * 16, wsb, None)
    assert call(3, 2) == K.KVQ_ERR_INVALID_ARG
    assert call(4, 0) == K.KVQ_ERR_INVALID_ARG
    assert call(4, 2, rot=K.KVQ_ROT_DENSE, R=None) == K.KVQ_ERR_INVALID_ARG   # dense needs R
    assert call(1, 4, wsb=100) == K.KVQ_ERR_WORKSPACE_TOO_SMALL


def test_varlen_bits_rejects(lib):
    """Per-sequence slots and ends at other code widths: the per-sequence
    arrays are required and 4-byte aligned; the width rules are those of
    the common-range calls."""
    def quant(kb, vb, offs=FAKE, dt=K.KVQ_F16, rot=K.KVQ_ROT_HADAMARD):
        return lib.kvq_quantize_at_bits(FAKE, FAKE, dt, 1, 8, 2, 128, 8 * 2 * 128, 2 * 128, 128,
                                        rot, None, 32, offs, ctypes.byref(_qcache(kb)),
                                        ctypes.byref(_qcache(vb)), None)
    assert quant(4, 2, offs=None) == K.KVQ_ERR_INVALID_ARG
    assert quant(4, 2, offs=FAKE + 2) == K.KVQ_ERR_INVALID_ARG
    assert quant(3, 2) == K.KVQ_ERR_INVALID_ARG
    assert quant(1, 1, dt=K.KVQ_F32) == K.KVQ_ERR_UNSUPPORTED
    assert quant(4, 2, rot=K.KVQ_ROT_NONE) == K.KVQ_ERR_UNSUPPORTED

    def dec(kb, vb, tends=FAKE, te_max=64, rot=K.KVQ_ROT_HADAMARD, R=None, wsb=1 << 30):
        return lib.kvq_decode_attention_varlen_bits(
            FAKE, K.KVQ_F16, 2, 4, 2, 128, ctypes.byref(_qcache(kb)), ctypes.byref(_qcache(vb)),
            0, tends, te_max, rot, R, 32, None, None, 0, None, None, 0, 0.0, FAKE, K.KVQ_F16,
            FAKE * 16, wsb, None)
    assert dec(4, 2, tends=None) == K.KVQ_ERR_INVALID_ARG
    assert dec(4, 2, tends=FAKE + 1) == K.KVQ_ERR_INVALID_ARG
    assert dec(2, 3) == K.KVQ_ERR_INVALID_ARG
    assert dec(4, 2, te_max=65) == K.KVQ_ERR_INVALID_ARG                 # beyond T_cap
    assert dec(1, 2, rot=K.KVQ_ROT_PERM_HADAMARD, R=None) == K.KVQ_ERR_INVALID_ARG   # no channel order
    assert dec(4, 4, wsb=100) == K.KVQ_ERR_WORKSPACE_TOO_SMALL


def _pcache(n_pages=4, page_tokens=128, bits=2):
    return K.kvq_paged_cache(FAKE, FAKE, FAKE, n_pages, page_tokens, bits)


def test_paged_rejects(lib):
    """Paged caches: pages of a multiple of 64 tokens, both sides alike, a
    4-byte aligned table; the write needs fp16 rows and a Hadamard rotation."""
    def dec(kc=None, vc=None, table=FAKE, maxp=4, te_max=512, tends=FAKE, wsb=1 << 30):
        kc = kc or _pcache()
        vc = vc or _pcache()
        return lib.kvq_decode_attention_paged(
            FAKE, K.KVQ_F16, 2, 4, 2, 128, ctypes.byref(kc), ctypes.byref(vc), 0, tends, te_max,
            table, maxp, K.KVQ_ROT_HADAMARD, None, 32, None, None, 0, None, None, 0, 0.0,
            FAKE, K.KVQ_F16, FAKE * 16, wsb, None)
    assert dec(kc=_pcache(page_tokens=96), vc=_pcache(page_tokens=96)) == K.KVQ_ERR_INVALID_ARG
    assert dec(vc=_pcache(n_pages=5)) == K.KVQ_ERR_INVALID_ARG          # sides differ
    assert dec(table=None) == K.KVQ_ERR_INVALID_ARG
    assert dec(table=FAKE + 2) == K.KVQ_ERR_INVALID_ARG
    assert dec(tends=None) == K.KVQ_ERR_INVALID_ARG
    assert dec(te_max=513) == K.KVQ_ERR_INVALID_ARG                      # beyond 4 pages x 128
    assert dec(wsb=100) == K.KVQ_ERR_WORKSPACE_TOO_SMALL
    assert dec(kc=_pcache(bits=3)) == K.KVQ_ERR_INVALID_ARG              # no 3-bit codes
    assert dec(vc=_pcache(bits=0)) == K.KVQ_ERR_INVALID_ARG

    def quant(dt=K.KVQ_F16, rot=K.KVQ_ROT_HADAMARD, offs=FAKE, R=None, kb=2, vb=2):
        return lib.kvq_quantize_paged(FAKE, FAKE, dt, 1, 8, 2, 128, 8 * 2 * 128, 2 * 128, 128,
                                      rot, R, 32, offs, FAKE, 4, ctypes.byref(_pcache(bits=kb)),
                                      ctypes.byref(_pcache(bits=vb)), None)
    assert quant(kb=4, vb=8) == K.KVQ_ERR_INVALID_ARG
    assert quant(kb=1, dt=K.KVQ_F32) == K.KVQ_ERR_UNSUPPORTED
    assert quant(kb=4, rot=K.KVQ_ROT_NONE) == K.KVQ_ERR_UNSUPPORTED
    assert quant(offs=None) == K.KVQ_ERR_INVALID_ARG
    # rows and rotations as for the contiguous caches
    assert quant(dt=K.KVQ_F32, rot=K.KVQ_ROT_DENSE, R=FAKE) == K.KVQ_ERR_UNSUPPORTED
    assert quant(dt=K.KVQ_F32, rot=K.KVQ_ROT_PERM_HADAMARD, R=FAKE) == K.KVQ_ERR_UNSUPPORTED
    assert quant(rot=K.KVQ_ROT_DENSE, R=None) == K.KVQ_ERR_INVALID_ARG


# ------------------------------------------------ pre-RoPE grouped-head keys
def _quant_prerope(lib, **kw):
    a = dict(K=FAKE, V=FAKE, dt=K.KVQ_F16, B=1, T=8, H=4, d=128, sb=8 * 4 * 128,
             st=4 * 128, sh=128, gh=4, group=32, toff=0, kc=_cache(), vc=_cache())
    a.update(kw)
    kc = ctypes.byref(a["kc"]) if a["kc"] is not None else None
    vc = ctypes.byref(a["vc"]) if a["vc"] is not None else None
    return lib.kvq_quantize_prerope(a["K"], a["V"], a["dt"], a["B"], a["T"], a["H"], a["d"],
                                    a["sb"], a["st"], a["sh"], a["gh"], a["group"], a["toff"],
                                    kc, vc, None)


@pytest.mark.parametrize("kw,want", [
    (dict(gh=3), K.KVQ_ERR_INVALID_ARG),
    (dict(gh=8), K.KVQ_ERR_INVALID_ARG),
    (dict(H=6, gh=4), K.KVQ_ERR_INVALID_ARG),              # heads not a multiple of the group
    (dict(H=6, gh=2, sb=8 * 6 * 128, st=6 * 128), K.KVQ_ERR_UNSUPPORTED),   # grouped: 4 heads per wave
    (dict(dt=K.KVQ_F32, sb=8 * 4 * 128, st=4 * 128), K.KVQ_ERR_UNSUPPORTED),
    (dict(d=64), K.KVQ_ERR_UNSUPPORTED),
    (dict(toff=60), K.KVQ_ERR_INVALID_ARG),
    (dict(K=None), K.KVQ_ERR_INVALID_ARG),
    (dict(kc=_cache(codes=0)), K.KVQ_ERR_INVALID_ARG),
])
def test_quantize_prerope_rejects(lib, kw, want):
    assert _quant_prerope(lib, **kw) == want


def test_quantize_prerope_empty_is_noop(lib):
    assert _quant_prerope(lib, T=0) == K.KVQ_OK
    assert _quant_prerope(lib, B=0, gh=1) == K.KVQ_OK


def _decode_prerope(lib, **kw):
    a = dict(q=FAKE, qdt=K.KVQ_F16, B=2, Hq=8, Hkv=4, d=128, kc=_cache(), vc=_cache(),
             tb=0, te=64, gh=4, base=10000.0, group=32, sk=None, sv=None, ns=0, rk=None,
             rv=None, nr=0, scale=0.0, out=FAKE, odt=K.KVQ_F16, ws=FAKE * 16, wsb=1 << 30)
    a.update(kw)
    kc = ctypes.byref(a["kc"]) if a["kc"] is not None else None
    vc = ctypes.byref(a["vc"]) if a["vc"] is not None else None
    return lib.kvq_decode_attention_prerope(a["q"], a["qdt"], a["B"], a["Hq"], a["Hkv"], a["d"],
                                            kc, vc, a["tb"], a["te"], a["gh"], a["base"], a["group"],
                                            a["sk"], a["sv"], a["ns"], a["rk"], a["rv"], a["nr"],
                                            a["scale"], a["out"], a["odt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(gh=3), K.KVQ_ERR_INVALID_ARG),
    (dict(Hkv=2, Hq=8), K.KVQ_ERR_INVALID_ARG),            # Hkv not a multiple of the group
    (dict(base=1.0), K.KVQ_ERR_INVALID_ARG),
    (dict(base=float("nan")), K.KVQ_ERR_INVALID_ARG),
    (dict(base=float("inf")), K.KVQ_ERR_INVALID_ARG),
    (dict(Hq=48, Hkv=4), K.KVQ_ERR_UNSUPPORTED),           # 4 x 12 query heads per group
    (dict(te=65), K.KVQ_ERR_INVALID_ARG),                  # past T_cap
    (dict(tb=5, te=4), K.KVQ_ERR_INVALID_ARG),
    (dict(wsb=100), K.KVQ_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws=FAKE + 16), K.KVQ_ERR_INVALID_ARG),           # workspace not 256-aligned
    (dict(d=256), K.KVQ_ERR_UNSUPPORTED),
])
def test_decode_prerope_rejects(lib, kw, want):
    assert _decode_prerope(lib, **kw) == want


def test_workspace_bytes_prerope():
    assert K.kvq_decode_workspace_bytes_prerope(0, 4, 4, 128, 10) == 0
    # one fp32 score per (b, query head, token) on top of the partials
    a = K.kvq_decode_workspace_bytes_prerope(2, 8, 4, 128, 1000)
    b = K.kvq_decode_workspace_bytes_prerope(2, 8, 4, 128, 1016)
    assert a >= 2 * 8 * 1000 * 4 and b - a >= 2 * 8 * 16 * 4
    assert K.kvq_decode_workspace_bytes_prerope(1, 4, 4, 128, 0, 4, 8) >= 0
