"""libaqua's C ABI without a GPU: the library loads, exports every call include/aqua.h declares,
and rejects bad arguments with the documented status before any HIP call (no pointer given
here is ever dereferenced)."""
import ctypes
import os
import re

import pytest

import sparse_dimension_attention_amd as aq
from sparse_dimension_attention_amd import aqua as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(aq.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return aq.load_library()


def _declared():
    with open(os.path.join(ROOT, "include", "aqua.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const char \*|aqua_status )(aqua_\w+)\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) == 16
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(aq.EXPORTS)
    assert "gfx950" in aq.aqua_version()


FAKE = 0x10000  # 16-byte aligned, never dereferenced


def _cache(**kw):
    c = dict(kp=FAKE, v=FAKE, B=2, Hkv=2, d_head=128, d_store=128, T_cap=256, len=10,
             dtype=A.AQUA_BF16)
    c.update(kw)
    return A.aqua_cache(**c)


def _decode(lib, cache, Hq=8, ws_bytes=1 << 30, q=FAKE, mask=FAKE, out=FAKE, ws=FAKE):
    return lib.aqua_decode(ctypes.byref(cache), Hq, q, mask, 0.1, None, out, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,Hq,status", [
    (dict(), 6, A.AQUA_ERR_SHAPE),                   # Hq not a multiple of Hkv
    (dict(), 2 * 16, A.AQUA_ERR_SHAPE),              # group size 16
    (dict(len=0), 8, A.AQUA_ERR_SHAPE),              # nothing to attend
    (dict(len=300), 8, A.AQUA_ERR_CAPACITY),         # len > T_cap
    (dict(T_cap=100), 8, A.AQUA_ERR_SHAPE),          # T_cap not a multiple of 64
    (dict(d_head=96), 8, A.AQUA_ERR_SHAPE),
    (dict(d_store=0), 8, A.AQUA_ERR_SHAPE),
    (dict(d_store=129), 8, A.AQUA_ERR_SHAPE),
    (dict(dtype=5), 8, A.AQUA_ERR_DTYPE),
    (dict(kp=None), 8, A.AQUA_ERR_NULL),
    (dict(v=FAKE + 8), 8, A.AQUA_ERR_ALIGN),
])
def test_decode_rejects(lib, kw, Hq, status):
    assert _decode(lib, _cache(**kw), Hq) == status
    assert lib.aqua_last_error().decode() != ""


def test_decode_rejects_buffers(lib):
    c = _cache()
    assert _decode(lib, c, q=None) == A.AQUA_ERR_NULL
    assert _decode(lib, c, ws=None) == A.AQUA_ERR_WORKSPACE
    assert _decode(lib, c, out=FAKE + 4) == A.AQUA_ERR_ALIGN
    need = ctypes.c_size_t(0)
    assert lib.aqua_decode_workspace(ctypes.byref(c), 8, ctypes.byref(need)) == A.AQUA_OK
    assert need.value > 0
    assert _decode(lib, c, ws_bytes=need.value - 1) == A.AQUA_ERR_WORKSPACE


def test_workspace_grows_with_capacity(lib):
    sizes = []
    for T_cap in (64, 2048, 8192, 131072):
        n = ctypes.c_size_t(0)
        assert lib.aqua_decode_workspace(ctypes.byref(_cache(T_cap=T_cap, len=1)), 8,
                                         ctypes.byref(n)) == A.AQUA_OK
        sizes.append(n.value)
    assert sizes == sorted(sizes) and sizes[0] > 0


def test_project_keys_rejects(lib):
    c = _cache(len=250)
    assert lib.aqua_project_keys(ctypes.byref(c), FAKE, FAKE, FAKE, 7, None, None) == \
        A.AQUA_ERR_CAPACITY
    assert c.len == 250
    assert lib.aqua_project_keys(ctypes.byref(c), None, FAKE, FAKE, 1, None, None) == \
        A.AQUA_ERR_NULL
    assert lib.aqua_project_keys(ctypes.byref(c), FAKE + 2, FAKE, FAKE, 1, None, None) == \
        A.AQUA_ERR_ALIGN
    assert lib.aqua_project_keys(ctypes.byref(c), FAKE, FAKE, FAKE, -1, None, None) == \
        A.AQUA_ERR_SHAPE
    # n == 0 is a no-op that touches nothing
    assert lib.aqua_project_keys(ctypes.byref(c), FAKE, FAKE, FAKE, 0, None, None) == A.AQUA_OK
    assert c.len == 250


@pytest.mark.parametrize("qdt,N,d,d_sel,k,status", [
    (A.AQUA_BF16, 4, 96, 96, 10, A.AQUA_ERR_SHAPE),
    (A.AQUA_BF16, 4, 128, 128, 0, A.AQUA_ERR_SHAPE),
    (A.AQUA_BF16, 4, 128, 64, 65, A.AQUA_ERR_SHAPE),
    (A.AQUA_BF16, 4, 128, 129, 96, A.AQUA_ERR_SHAPE),
    (A.AQUA_BF16, -1, 128, 128, 96, A.AQUA_ERR_SHAPE),
    (7, 4, 128, 128, 96, A.AQUA_ERR_DTYPE),
    (A.AQUA_F32, 0, 128, 128, 96, A.AQUA_OK),  # empty: no-op
])
def test_select_rejects(lib, qdt, N, d, d_sel, k, status):
    assert lib.aqua_select_dims(FAKE, qdt, N, d, FAKE, d_sel, k, FAKE, FAKE, None, None) == status


def test_h2o_victim_rejects(lib):
    assert lib.aqua_h2o_victim(None, FAKE, 1, 1, 4, 10, 2, FAKE, None) == A.AQUA_ERR_NULL
    assert lib.aqua_h2o_victim(FAKE, FAKE, 1, 1, 0, 10, 2, FAKE, None) == A.AQUA_ERR_SHAPE
    assert lib.aqua_h2o_victim(FAKE, FAKE, 1, 1, 4, 10, -1, FAKE, None) == A.AQUA_ERR_SHAPE
    assert lib.aqua_h2o_victim(FAKE + 4, FAKE, 1, 1, 4, 10, 2, FAKE, None) == A.AQUA_ERR_ALIGN
    assert lib.aqua_h2o_victim(FAKE, FAKE + 8, 1, 1, 4, 10, 2, FAKE, None) == A.AQUA_ERR_ALIGN
    assert lib.aqua_h2o_victim(FAKE, FAKE, 1, 1, 4, 10, 2, FAKE + 4, None) == A.AQUA_ERR_ALIGN


def _h2o_init(lib, full, compact, heavy=1024, recent=256, mass_full=FAKE, mass=FAKE,
              slot_pos=FAKE):
    return lib.aqua_h2o_init(ctypes.byref(full), mass_full, heavy, recent, ctypes.byref(compact),
                             mass, slot_pos, None)


@pytest.mark.parametrize("fkw,ckw,args,status", [
    (dict(), dict(), dict(mass=None), A.AQUA_ERR_NULL),
    (dict(), dict(), dict(mass_full=FAKE + 4), A.AQUA_ERR_ALIGN),
    (dict(), dict(), dict(slot_pos=FAKE + 8), A.AQUA_ERR_ALIGN),
    (dict(), dict(d_store=128), dict(), A.AQUA_ERR_SHAPE),         # d_store differs
    (dict(), dict(dtype=A.AQUA_F32), dict(), A.AQUA_ERR_SHAPE),    # dtype differs
    (dict(), dict(B=2), dict(), A.AQUA_ERR_SHAPE),                 # batch differs
    (dict(), dict(len=1200), dict(), A.AQUA_ERR_SHAPE),            # compact cache not full
    (dict(), dict(), dict(heavy=1000), A.AQUA_ERR_SHAPE),          # T_cap != heavy + recent
    (dict(), dict(), dict(heavy=-64, recent=1344), A.AQUA_ERR_SHAPE),
    (dict(len=1000), dict(), dict(), A.AQUA_ERR_CAPACITY),         # fewer tokens than slots
    (dict(d_head=96), dict(), dict(), A.AQUA_ERR_SHAPE),
])
def test_h2o_init_rejects(lib, fkw, ckw, args, status):
    full = _cache(**dict(dict(B=1, Hkv=8, d_store=96, T_cap=32768, len=32768), **fkw))
    compact = _cache(**dict(dict(B=1, Hkv=8, d_store=96, T_cap=1280, len=1280), **ckw))
    assert _h2o_init(lib, full, compact, **args) == status
    assert lib.aqua_last_error().decode() != ""


def test_binding_raises_with_message(lib):
    with pytest.raises(aq.AquaError, match="AQUA_ERR_SHAPE"):
        A._check(_decode(lib, _cache(len=0)))


def _prefill(lib, cache, Hq=8, Lq=4, pos0=0, d_sel=128, k=96, q=FAKE, P=FAKE, out=FAKE, ws=FAKE,
             ws_bytes=1 << 30, q_proj=None):
    return lib.aqua_prefill_chunk(ctypes.byref(cache), Hq, q, Lq, pos0, P, d_sel, k, 0.1, out,
                                  q_proj, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,args,status", [
    (dict(dtype=A.AQUA_F32), dict(), A.AQUA_ERR_DTYPE),      # prefill is bf16 only
    (dict(d_head=64, d_store=64), dict(), A.AQUA_ERR_SHAPE),  # and d_head 128 only
    (dict(d_store=100), dict(d_sel=96), A.AQUA_ERR_SHAPE),    # d_store a multiple of 16
    (dict(), dict(Hq=6), A.AQUA_ERR_SHAPE),                   # Hq not a multiple of Hkv
    (dict(), dict(q=None), A.AQUA_ERR_NULL),
    (dict(), dict(ws=None), A.AQUA_ERR_WORKSPACE),
    (dict(), dict(Lq=0), A.AQUA_ERR_SHAPE),
    (dict(), dict(pos0=-1), A.AQUA_ERR_SHAPE),
    (dict(), dict(pos0=8, Lq=4), A.AQUA_ERR_CAPACITY),        # pos0 + Lq > len = 10
    (dict(), dict(k=0), A.AQUA_ERR_SHAPE),
    (dict(), dict(k=97, d_sel=96), A.AQUA_ERR_SHAPE),         # k > d_sel
    (dict(d_store=96), dict(d_sel=128), A.AQUA_ERR_SHAPE),    # d_sel > d_store
    (dict(), dict(out=FAKE + 4), A.AQUA_ERR_ALIGN),
    (dict(), dict(q_proj=FAKE + 8), A.AQUA_ERR_ALIGN),
    (dict(), dict(ws_bytes=16), A.AQUA_ERR_WORKSPACE),
])
def test_prefill_rejects(lib, kw, args, status):
    assert _prefill(lib, _cache(**kw), **args) == status
    assert lib.aqua_last_error().decode() != ""


def _step(lib, cache, Hq=8, d_sel=128, k=96, q=FAKE, k_new=FAKE, out=FAKE, ws=FAKE,
          ws_bytes=1 << 30, mass=None):
    return lib.aqua_decode_step(ctypes.byref(cache), Hq, q, k_new, FAKE, FAKE, d_sel, k, 0.1,
                                mass, out, None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,args,status", [
    (dict(), dict(Hq=6), A.AQUA_ERR_SHAPE),
    (dict(len=256), dict(), A.AQUA_ERR_CAPACITY),  # no column left for the new token
    (dict(), dict(k_new=None), A.AQUA_ERR_NULL),
    (dict(), dict(ws=None), A.AQUA_ERR_WORKSPACE),
    (dict(), dict(k=0), A.AQUA_ERR_SHAPE),
    (dict(d_store=96), dict(d_sel=128), A.AQUA_ERR_SHAPE),
    (dict(), dict(mass=FAKE + 4), A.AQUA_ERR_ALIGN),
    (dict(), dict(ws_bytes=16), A.AQUA_ERR_WORKSPACE),
])
def test_decode_step_rejects(lib, kw, args, status):
    c = _cache(**kw)
    assert _step(lib, c, **args) == status
    assert c.len == kw.get("len", 10)  # a rejected step appends nothing


def _h2o_step(lib, cache, Hq=8, k=64, t_new=300, recent=16, mass=FAKE, slot_pos=FAKE,
              victim=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.aqua_h2o_step(ctypes.byref(cache), Hq, FAKE, FAKE, FAKE, FAKE, 96, k, 0.1, mass,
                             slot_pos, t_new, recent, victim, FAKE, None, None, ws, ws_bytes,
                             None)


@pytest.mark.parametrize("kw,args,status", [
    (dict(len=200), dict(), A.AQUA_ERR_SHAPE),        # the compact cache must be full
    (dict(T_cap=8192, len=8192), dict(), A.AQUA_ERR_SHAPE),  # more slots than the fused step takes
    (dict(), dict(mass=None), A.AQUA_ERR_NULL),
    (dict(), dict(victim=None), A.AQUA_ERR_NULL),
    (dict(), dict(ws=None), A.AQUA_ERR_WORKSPACE),
    (dict(), dict(k=97), A.AQUA_ERR_SHAPE),           # k > d_sel = 96
    (dict(), dict(recent=-1), A.AQUA_ERR_SHAPE),
    (dict(), dict(mass=FAKE + 4), A.AQUA_ERR_ALIGN),
    (dict(), dict(ws_bytes=16), A.AQUA_ERR_WORKSPACE),
])
def test_h2o_step_rejects(lib, kw, args, status):
    c = _cache(**dict(dict(d_store=96, T_cap=256, len=256), **kw))
    assert _h2o_step(lib, c, **args) == status


@pytest.mark.parametrize("kw,args,status", [
    (dict(), dict(Hq=6), A.AQUA_ERR_SHAPE),
    (dict(len=256), dict(), A.AQUA_ERR_CAPACITY),
    (dict(), dict(q=None), A.AQUA_ERR_NULL),
    (dict(), dict(k=0), A.AQUA_ERR_SHAPE),
    (dict(), dict(out=FAKE + 4), A.AQUA_ERR_ALIGN),
    # more workspace than the 32 MiB static scratch: 64 x 128 heads x 8192 tokens of scores
    (dict(B=64, Hkv=32, T_cap=8192, len=100), dict(Hq=128, mass=FAKE), A.AQUA_ERR_WORKSPACE),
])
def test_decode_step_noalloc_rejects(lib, kw, args, status):
    c = _cache(**kw)
    a = dict(Hq=8, q=FAKE, k=96, out=FAKE, mass=None)
    a.update(args)
    assert lib.aqua_decode_step_noalloc(ctypes.byref(c), a["Hq"], a["q"], FAKE, FAKE, FAKE, 128,
                                        a["k"], 0.1, a["mass"], a["out"], None, None,
                                        None) == status
    assert lib.aqua_last_error().decode() != ""
    assert c.len == kw.get("len", 10)


def test_stream_read_probe_rejects(lib):
    assert lib.aqua_stream_read_probe(None, 1024, 4, FAKE, None) == A.AQUA_ERR_NULL
    assert lib.aqua_stream_read_probe(FAKE, 1000, 4, FAKE, None) == A.AQUA_ERR_SHAPE
    assert lib.aqua_stream_read_probe(FAKE, 1024, 0, FAKE, None) == A.AQUA_ERR_SHAPE
    assert lib.aqua_stream_read_probe(FAKE + 4, 1024, 4, FAKE, None) == A.AQUA_ERR_ALIGN


def test_gram_rejects(lib):
    nb = ctypes.c_size_t()
    assert lib.aqua_gram_workspace(A.AQUA_BF16, 1000, 128, ctypes.byref(nb)) == A.AQUA_OK
    assert nb.value == 8 * 128 * 128 * 4  # eight 128-row chunks of fp32 partials
    assert lib.aqua_gram_workspace(A.AQUA_BF16, 1000, 96, ctypes.byref(nb)) == A.AQUA_ERR_SHAPE
    assert lib.aqua_gram_workspace(7, 1000, 128, ctypes.byref(nb)) == A.AQUA_ERR_DTYPE
    assert lib.aqua_gram_workspace(A.AQUA_F32, 0, 64, ctypes.byref(nb)) == A.AQUA_ERR_SHAPE
    assert lib.aqua_gram_workspace(A.AQUA_F32, 10, 64, None) == A.AQUA_ERR_NULL
    big = 1 << 24
    assert lib.aqua_gram(A.AQUA_F32, None, 10, 64, FAKE, FAKE, big, None) == A.AQUA_ERR_NULL
    assert lib.aqua_gram(A.AQUA_F32, FAKE, 10, 64, None, FAKE, big, None) == A.AQUA_ERR_NULL
    assert lib.aqua_gram(A.AQUA_F32, FAKE + 4, 10, 64, FAKE, FAKE, big, None) == A.AQUA_ERR_ALIGN
    assert lib.aqua_gram(A.AQUA_F32, FAKE, 10, 64, FAKE, FAKE, 100, None) == A.AQUA_ERR_WORKSPACE
    assert lib.aqua_gram(A.AQUA_BF16, FAKE, 10, 32, FAKE, FAKE, big, None) == A.AQUA_ERR_SHAPE
