"""Host-side checks of the C ABI (CPU only: no kernel is launched).

The library must load, export every function include/rocketkv.h declares,
compute the split exactly as the oracle does, and reject bad arguments with
the documented codes before touching the device.
"""

import ctypes
import os
import re

import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rocketkv.h")
LIB = os.path.join(ROOT, "sparse_decode_attention_amd", "librocketkv.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="librocketkv.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rk_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"rk_split", "rk_snapkv_evict", "rk_hsa_build_aux", "rk_hsa_decode",
            "rk_hsa_decode_mt", "rk_append_kv", "rk_hsa_append_decode"} <= set(names)
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    nm = os.popen(f"nm -D --defined-only {LIB}").read()
    for n in names:
        assert re.search(rf"\bT {n}$", nm, flags=re.M), f"{n} not exported as a C symbol"


@pytest.fixture(scope="module")
def rk():
    from sparse_decode_attention_amd import rocketkv
    return rocketkv


@pytest.mark.parametrize("c,S,W,B,d", [(8, 2048, 16, 16, 64), (16, 32768, 32, 16, 128),
                                       (64, 32768, 32, 16, 128), (109568 / 256, 109568, 32, 16, 128),
                                       (32, 33792, 32, 16, 128), (32, 36864, 32, 16, 128),
                                       (1, 100, 10, 16, 64), (1e7, 100, 10, 16, 64), (2 ** 10, 5000, 7, 3, 96)])
def test_split_matches_oracle(rk, c, S, W, B, d):
    got = rk.rk_split(c, S, W, B, d)
    want = O.split(c, S, W, B, d)
    for key in ("r", "c1", "c2", "budget_t", "paper_k1"):
        assert got[key] == pytest.approx(want[key], rel=1e-12), key
    for key in ("n_keep", "k2_blocks", "paper_page", "paper_k1_channels", "paper_k2_blocks"):
        assert got[key] == want[key], key


def test_split_config_values(rk):
    """Keep counts and page budgets of the workloads (readings R2, R3)."""
    assert rk.rk_split(8, 2048, 16, 16, 64)["n_keep"] == 930
    s = rk.rk_split(16, 32768, 32, 16, 128)
    assert (s["n_keep"], s["k2_blocks"]) == (9675, 128)
    s = rk.rk_split(64, 32768, 32, 16, 128)
    assert (s["n_keep"], s["k2_blocks"]) == (3192, 32)
    s = rk.rk_split(428, 109568, 32, 16, 128)
    assert (s["n_keep"], s["k2_blocks"]) == (1360, 16) and round(s["r"], 2) == 0.72
    assert [rk.rk_split(32, 32768 + 1024 * t, 32, 16, 128)["n_keep"] for t in range(1, 5)] == \
        [5974, 6155, 6336, 6517]


def test_split_rejects(rk):
    with pytest.raises(rk.RocketKVError) as e:
        rk.rk_split(0.5, 100, 10, 16, 64)
    assert e.value.status == rk.RK_EINVAL
    with pytest.raises(rk.RocketKVError):
        rk.rk_split(4, 100, 101, 16, 64)
    with pytest.raises(rk.RocketKVError):
        rk.rk_split(4, 100, 10, 0, 64)
    lib = rk.raw_library()
    assert lib.rk_split(4.0, 100, 10, 16, 64, None) == rk.RK_EINVAL


FAKE = 1 << 20   # a non-null, aligned address that is never dereferenced


def _vp(x):
    return ctypes.c_void_p(x)


def test_error_codes_before_any_launch(rk):
    lib = rk.raw_library()
    sh = rk.shape_of(1, 8, 2, 64, rk.RK_F32)
    byref = ctypes.byref

    def decode(**kw):
        a = dict(shape=byref(sh), q=_vp(FAKE), k=_vp(FAKE), v=_vp(FAKE), cap=1024, kmax=_vp(FAKE),
                 kmin=_vp(FAKE), nblk_cap=64, n=1000, block=16, k1=16, k2=16, out=_vp(FAKE),
                 ws=_vp(FAKE), ws_bytes=1 << 30)
        a.update(kw)
        return lib.rk_hsa_decode(a["shape"], a["q"], a["k"], a["v"], a["cap"], a["kmax"], a["kmin"],
                                 a["nblk_cap"], a["n"], a["block"], a["k1"], a["k2"], a["out"],
                                 None, None, None, a["ws"], a["ws_bytes"], None)

    assert decode(shape=None) == rk.RK_EINVAL
    assert decode(q=None) == rk.RK_EINVAL
    assert decode(q=_vp(FAKE + 4)) == rk.RK_EINVAL                   # misaligned
    assert decode(k1=0) == rk.RK_EINVAL and decode(k1=65) == rk.RK_EINVAL
    assert decode(k2=0) == rk.RK_EINVAL
    assert decode(n=0) == rk.RK_EINVAL and decode(n=1025) == rk.RK_EINVAL
    assert decode(nblk_cap=62) == rk.RK_EINVAL
    assert decode(nblk_cap=66) == rk.RK_EINVAL                         # not a multiple of 8
    assert decode(block=0) == rk.RK_EINVAL
    assert decode(ws_bytes=16) == rk.RK_EWORKSPACE
    assert b"workspace" in lib.rk_last_error()
    assert decode(ws=_vp(FAKE + 64)) == rk.RK_EINVAL                 # not 256-aligned
    bad_heads = rk.shape_of(1, 6, 4, 64, rk.RK_F32)
    assert decode(shape=byref(bad_heads)) == rk.RK_EINVAL
    g3 = rk.shape_of(1, 6, 2, 64, rk.RK_F32)
    assert decode(shape=byref(g3)) == rk.RK_EUNSUPPORTED
    d96 = rk.shape_of(1, 8, 2, 96, rk.RK_F32)
    assert decode(shape=byref(d96)) == rk.RK_EUNSUPPORTED
    big = rk.shape_of(1, 8, 2, 64, rk.RK_F32)
    # more pages than the decode path takes (2^22)
    assert decode(shape=byref(big), n=(1 << 22) + 1, cap=(1 << 22) + 1, block=1,
                  nblk_cap=(1 << 22) + 8) == rk.RK_EUNSUPPORTED

    def evict(**kw):
        a = dict(q=_vp(FAKE), k=_vp(FAKE), v=_vp(FAKE), cap=2048, S=2048, W=16, pool=7, keep=930,
                 kept=_vp(FAKE), ko=_vp(FAKE), vo=_vp(FAKE), out_cap=930, ws=_vp(FAKE), wsb=1 << 30,
                 kmax=None, kmin=None, nblk_cap=0, block=16)
        a.update(kw)
        return lib.rk_snapkv_evict(byref(sh), a["q"], a["k"], a["v"], a["cap"], a["S"], a["W"],
                                   a["pool"], a["keep"], a["kept"], a["ko"], a["vo"], a["out_cap"],
                                   None, a["kmax"], a["kmin"], a["nblk_cap"], a["block"], a["ws"],
                                   a["wsb"], None)

    assert evict(pool=8) == rk.RK_EINVAL and evict(pool=0) == rk.RK_EINVAL
    assert evict(keep=15) == rk.RK_EINVAL and evict(keep=2049) == rk.RK_EINVAL
    assert evict(W=0) == rk.RK_EINVAL and evict(W=2049) == rk.RK_EINVAL
    assert evict(S=4096) == rk.RK_EINVAL                                # above kv_cap
    assert evict(out_cap=929) == rk.RK_EINVAL
    assert evict(vo=None) == rk.RK_EINVAL                               # k_out without v_out
    assert evict(kmax=_vp(FAKE)) == rk.RK_EINVAL                        # kmax without kmin
    aux = dict(kmax=_vp(FAKE), kmin=_vp(FAKE), nblk_cap=64)
    assert evict(**aux, block=0) == rk.RK_EINVAL
    assert evict(**dict(aux, nblk_cap=56)) == rk.RK_EINVAL               # 930 tokens need 59 pages
    assert evict(**dict(aux, nblk_cap=60)) == rk.RK_EINVAL               # not a multiple of 8
    assert evict(**aux, ko=None, vo=None) == rk.RK_EINVAL                # aux needs the compact cache
    assert evict(wsb=100) == rk.RK_EWORKSPACE
    need = lib.rk_snapkv_workspace_bytes(byref(sh), 2048, 16)
    assert need > 0 and evict(wsb=need - 1) == rk.RK_EWORKSPACE

    def evict_pool(op, **kw):
        a = dict(pool=7, keep=930, wsb=1 << 30)
        a.update(kw)
        return lib.rk_snapkv_evict_pool(byref(sh), _vp(FAKE), _vp(FAKE), _vp(FAKE), 2048, 2048, 16,
                                        a["pool"], op, a["keep"], _vp(FAKE), _vp(FAKE), _vp(FAKE), 930,
                                        None, None, None, 0, 16, _vp(FAKE), a["wsb"], None)

    assert evict_pool(2) == rk.RK_EINVAL and evict_pool(-1) == rk.RK_EINVAL   # no such pooling
    assert b"pool_op" in lib.rk_last_error()
    assert evict_pool(1, pool=8) == rk.RK_EINVAL
    assert evict_pool(1, wsb=100) == rk.RK_EWORKSPACE                         # max pooling passes the checks
    ada = lib.rk_adakv_evict_pool(byref(sh), _vp(FAKE), _vp(FAKE), _vp(FAKE), 2048, 2048, 16, 7, 5, 930,
                                  _vp(FAKE), _vp(FAKE), _vp(FAKE), _vp(FAKE), 2048, None, None, None, 0, 16,
                                  _vp(FAKE), 1 << 30, None)
    assert ada == rk.RK_EINVAL and b"pool_op" in lib.rk_last_error()

    def aux(**kw):
        a = dict(k=_vp(FAKE), cap=1024, idx=None, stride=0, n=1000, first=0, block=16, nblk_cap=64)
        a.update(kw)
        return lib.rk_hsa_build_aux(byref(sh), a["k"], a["cap"], a["idx"], a["stride"], a["n"],
                                    a["first"], a["block"], _vp(FAKE), _vp(FAKE), a["nblk_cap"], None)

    assert aux(nblk_cap=62) == rk.RK_EINVAL
    assert aux(nblk_cap=63) == rk.RK_EINVAL                            # not a multiple of 8
    assert aux(first=1000) == rk.RK_EINVAL and aux(first=-1) == rk.RK_EINVAL
    assert aux(n=1025) == rk.RK_EINVAL
    assert aux(idx=_vp(FAKE), stride=999) == rk.RK_EINVAL
    assert aux(k=None) == rk.RK_EINVAL

    def app(**kw):
        a = dict(kn=_vp(FAKE), cap=1024, pos=1000, nblk_cap=64, block=16)
        a.update(kw)
        return lib.rk_append_kv(byref(sh), a["kn"], _vp(FAKE), _vp(FAKE), _vp(FAKE), a["cap"], a["pos"],
                                _vp(FAKE), _vp(FAKE), a["nblk_cap"], a["block"], None)

    assert app(pos=1024) == rk.RK_EINVAL and app(pos=-1) == rk.RK_EINVAL
    assert app(nblk_cap=62) == rk.RK_EINVAL and app(nblk_cap=63) == rk.RK_EINVAL
    assert app(kn=None) == rk.RK_EINVAL and app(block=0) == rk.RK_EINVAL

    def appdec(**kw):
        a = dict(kn=_vp(FAKE), vn=_vp(FAKE), cap=1024, pos=999, nblk_cap=64, block=16)
        a.update(kw)
        return lib.rk_hsa_append_decode(byref(sh), _vp(FAKE), a["kn"], a["vn"], _vp(FAKE), _vp(FAKE),
                                        a["cap"], a["pos"], _vp(FAKE), _vp(FAKE), a["nblk_cap"],
                                        a["block"], 16, 16, _vp(FAKE), None, None, None, _vp(FAKE),
                                        1 << 30, None)

    assert appdec(pos=-1) == rk.RK_EINVAL and appdec(pos=1024) == rk.RK_EINVAL
    assert appdec(kn=None) == rk.RK_EINVAL and appdec(vn=None) == rk.RK_EINVAL
    assert appdec(kn=_vp(FAKE + 2)) == rk.RK_EINVAL                    # misaligned
    assert appdec(nblk_cap=56) == rk.RK_EINVAL                          # 1000 tokens need 63 pages
    assert appdec(block=0) == rk.RK_EINVAL

    assert lib.rk_hsa_decode_mt(byref(sh), _vp(FAKE), _vp(FAKE), _vp(FAKE), 4096, None, 1000, 1000,
                                _vp(FAKE), _vp(FAKE), 63, 16, 16, 16, _vp(FAKE), None, None, None,
                                _vp(FAKE), 1 << 30, None) == rk.RK_EINVAL
    for s in range(5):
        assert lib.rk_status_string(s).startswith(b"RK_")


def test_workspace_sizes_monotone(rk):
    lib = rk.raw_library()
    sh = rk.shape_of(4, 32, 8, 128, rk.RK_BF16)
    a = lib.rk_snapkv_workspace_bytes(ctypes.byref(sh), 4096, 32)
    b = lib.rk_snapkv_workspace_bytes(ctypes.byref(sh), 8192, 32)
    assert 0 < a < b and a % 256 == 0
    c = lib.rk_hsa_workspace_bytes(ctypes.byref(sh), 3000, 16, 32, 32)
    e = lib.rk_hsa_workspace_bytes(ctypes.byref(sh), 3000, 16, 32, 64)
    assert 0 < c < e
    assert lib.rk_hsa_workspace_bytes(ctypes.byref(sh), 0, 16, 32, 32) == 0
    assert lib.rk_snapkv_workspace_bytes(None, 4096, 32) == 0


def test_noalloc_refuses_oversized_call_before_the_device(rk):
    """rk_hsa_decode_noalloc checks its scratch need first: a call larger than
    the static scratch returns RK_EWORKSPACE without touching a device (this
    runs where there is none)."""
    lib = rk.raw_library()
    assert lib.rk_hsa_decode_noalloc_max_bytes() == 16 << 20
    shape = rk.shape_of(64, 32, 8, 128, rk.RK_BF16)
    n = 12000 * 16
    assert rk.rk_hsa_workspace_bytes(shape, n, 16, 32, 256) > 16 << 20
    fake = ctypes.c_void_p(1 << 20)
    st = lib.rk_hsa_decode_noalloc(ctypes.byref(shape), fake, fake, fake, n, fake, fake, 12000, n, 16, 32,
                                   256, fake, None, None, None, None)
    assert st == rk.RK_EWORKSPACE
    assert b"static scratch" in lib.rk_last_error()


@pytest.mark.parametrize("method", ["hsa", "quest", "sparq", "exact"])
@pytest.mark.parametrize("c,S,d", [(16, 32768, 128), (109568 / 256, 109568, 128), (4, 4096, 64),
                                   (1, 100, 64), (1000, 5000, 128)])
def test_select_plan_matches_oracle(rk, method, c, S, d):
    got = rk.rk_select_plan(method, c, S, d)
    want = O.select_plan(method, c, S, d)
    for key in ("page", "channels", "k2", "attn_tokens"):
        assert got[key] == want[key], key
    for key in ("budget_t", "est_pairs"):
        assert got[key] == pytest.approx(want[key], rel=1e-12), key


def test_select_decode_rejects_before_any_launch(rk):
    lib = rk.raw_library()
    sh = rk.shape_of(1, 8, 2, 64, rk.RK_BF16)
    f = _vp(FAKE)

    def call(method, page, channels, kmax=f):
        return lib.rk_select_decode(ctypes.byref(sh), method, f, f, f, 4096, kmax, kmax, 4096, 4000, page,
                                    channels, 64, f, None, None, f, 16, None)   # tiny workspace

    assert call(1, 16, 32) == rk.RK_EINVAL          # Quest needs every channel
    assert call(2, 4, 8) == rk.RK_EINVAL            # SparQ needs pages of one token
    assert call(3, 1, 32) == rk.RK_EINVAL           # Exact needs every channel
    assert call(3, 2, 64) == rk.RK_EINVAL           # and pages of one token
    assert call(7, 1, 64) == rk.RK_EINVAL           # unknown method
    assert call(3, 1, 64, kmax=None) == rk.RK_EWORKSPACE   # exact ignores the aux; workspace too small
    assert lib.rk_select_plan(0, 0.5, 100, 64, None) == rk.RK_EINVAL


def test_paged_descriptor_checked_before_any_launch(rk):
    lib = rk.raw_library()
    sh = rk.shape_of(1, 8, 2, 128, rk.RK_BF16)
    f = _vp(FAKE)

    def dec(P=64, n_pages=16, stride=4, table=FAKE, shape=sh, n=200):
        pk = rk.RkPagedKv(table, stride, n_pages, P)
        return lib.rk_paged_hsa_decode(ctypes.byref(shape), f, f, f, ctypes.byref(pk), f, f, 16, n, 16, 16, 8, f,
                                       None, None, None, f, 16, None)

    assert dec() == rk.RK_EWORKSPACE                  # descriptor fine, workspace too small
    assert dec(P=48) == rk.RK_EINVAL                  # not a power of two
    assert dec(P=0) == rk.RK_EINVAL
    assert dec(table=None) == rk.RK_EINVAL
    assert dec(table=FAKE + 2) == rk.RK_EINVAL        # misaligned table
    assert dec(n=257) == rk.RK_EINVAL                 # beyond the 4 pages of 64 of the table row
    assert dec(n_pages=0) == rk.RK_EINVAL
    assert dec(n_pages=1 << 26) == rk.RK_EUNSUPPORTED  # 2^31 pool rows or more
    f32 = rk.shape_of(1, 8, 2, 128, rk.RK_F32)
    assert dec(shape=f32) == rk.RK_EUNSUPPORTED        # bf16 only
    assert lib.rk_paged_hsa_decode(ctypes.byref(sh), f, f, f, None, f, f, 16, 200, 16, 16, 8, f, None, None,
                                   None, f, 1 << 20, None) == rk.RK_EINVAL


def test_binding_refuses_host_tensors_and_wrong_types(rk):
    """The binding stops a host tensor (whose address a kernel would fault on)
    and index / output tensors of the wrong element type before the library
    is called."""
    import torch
    k = torch.zeros(1, 2, 64, 64)
    kmax = torch.zeros(1, 2, 64, 8)
    with pytest.raises(ValueError, match="on the GPU"):
        rk.rk_hsa_build_aux(k, 64, 0, 16, kmax, kmax.clone())
    with pytest.raises(TypeError):
        rk.rk_hsa_build_aux(k, 64, 0, 16, kmax.to(torch.bfloat16), kmax.clone())
    with pytest.raises(TypeError):
        rk.rk_hsa_build_aux(k, 64, 0, 16, kmax, kmax.clone(), idx=torch.zeros(1, 2, 64, dtype=torch.int64))
    q = torch.zeros(1, 4, 64)
    with pytest.raises(TypeError):   # the output is float32
        rk.rk_hsa_decode(q, k, k, kmax, kmax, 64, 16, 16, 4, torch.zeros(1, 4, 64, dtype=torch.float64))
    with pytest.raises(TypeError):   # indices are int32
        rk.rk_hsa_decode(q, k, k, kmax, kmax, 64, 16, 16, 4, torch.zeros(1, 4, 64),
                         sel_blocks=torch.zeros(1, 2, 4, dtype=torch.int64))
    with pytest.raises(TypeError):   # the paged block table is int32
        rk.paged_kv(torch.zeros(1, 4, dtype=torch.int64), 4, 16)
