"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and its host-side validation returns the documented status
for each bad argument (nothing is launched on those paths)."""
import ctypes
import os
import re
import subprocess

import pytest

from quantized_mixture_experts_moe_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ops.LIB_PATH),
                                reason="libqmoe.so not built (run __graft_entry__.build())")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmoe_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert _declared() == sorted(ops.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ops.lib()
    nm = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True,
                        text=True).stdout
    for name in _declared():
        assert hasattr(L, name), name
        assert re.search(rf"\bT {name}$", nm, flags=re.M), name


def test_version_and_status_strings():
    L = ops.lib()
    assert L.qmoe_abi_version() == 4 == ops.ABI_VERSION
    for s in range(4):
        assert L.qmoe_status_str(s)
    assert L.qmoe_status_str(99) == b"unknown status"


def test_align_capacity_formula():
    L = ops.lib()
    for T, k, E, bm in [(64, 2, 8, 16), (128, 8, 128, 16), (4096, 10, 512, 128), (1, 1, 1, 64),
                        (0, 4, 8, 32), (8192, 10, 512, 128)]:
        P = T * k
        cap = P + min(E, P) * (bm - 1)
        cap = max(cap, 1)
        cap = (cap + bm - 1) // bm * bm
        assert L.qmoe_align_capacity(T, k, E, bm) == cap
    assert L.qmoe_align_capacity(4, 2, 8, 48) == 0  # unsupported block_m


def test_route_validation():
    L = ops.lib()
    p = ctypes.c_void_p(0x1000)
    assert L.qmoe_route(p, 4, 8, 9, p, p, None) == ops.QMOE_ERR_INVALID_ARG  # k > E
    assert L.qmoe_route(p, 4, 64, 17, p, p, None) == ops.QMOE_ERR_INVALID_ARG  # k > 16
    assert L.qmoe_route(p, 4, 2048, 8, p, p, None) == ops.QMOE_ERR_UNSUPPORTED
    assert L.qmoe_route(None, 4, 8, 2, p, p, None) == ops.QMOE_ERR_INVALID_ARG
    assert L.qmoe_route(None, 0, 8, 2, None, None, None) == ops.QMOE_OK  # T = 0: nothing to do


def test_align_validation():
    L = ops.lib()
    p = ctypes.c_void_p(0x1000)
    ws = L.qmoe_align_workspace(64, 2, 8)
    assert ws >= 256
    assert L.qmoe_align(p, 64, 2, 8, 24, p, p, p, p, p, ws, None) == ops.QMOE_ERR_INVALID_ARG
    assert L.qmoe_align(p, 64, 9, 8, 16, p, p, p, p, p, ws, None) == ops.QMOE_ERR_INVALID_ARG
    assert L.qmoe_align(None, 64, 2, 8, 16, p, p, p, p, p, ws, None) == ops.QMOE_ERR_INVALID_ARG
    assert L.qmoe_align(p, 64, 2, 8, 16, p, p, p, p, p, ws - 1, None) == ops.QMOE_ERR_INVALID_ARG
    assert L.qmoe_align(p, 64, 2, 2000, 16, p, p, p, p, p, 1 << 30, None) == \
        ops.QMOE_ERR_UNSUPPORTED
    assert L.qmoe_check_flags(None, None, None) == ops.QMOE_ERR_INVALID_ARG


def test_route_align_validation():
    """qmoe_route_align checks what qmoe_route and qmoe_align check."""
    L = ops.lib()
    p = ctypes.c_void_p(0x1000)
    ws = L.qmoe_align_workspace(16, 4, 64)
    ok = dict(T=16, E=64, k=4, bm=16)

    def call(T=16, E=64, k=4, bm=16, logits=p, ids=p, w=p, srt=p, wsp=p, wsb=ws):
        return L.qmoe_route_align(logits, T, E, k, bm, ids, w, srt, p, p, p, wsp, wsb, None)
    assert call(bm=24) == ops.QMOE_ERR_INVALID_ARG
    assert call(k=17, E=64) == ops.QMOE_ERR_INVALID_ARG
    assert call(k=65) == ops.QMOE_ERR_INVALID_ARG
    assert call(T=-1) == ops.QMOE_ERR_INVALID_ARG
    assert call(logits=None) == ops.QMOE_ERR_INVALID_ARG
    assert call(w=None) == ops.QMOE_ERR_INVALID_ARG
    assert call(srt=None) == ops.QMOE_ERR_INVALID_ARG
    assert call(wsp=None) == ops.QMOE_ERR_INVALID_ARG
    assert call(wsb=ws - 1) == ops.QMOE_ERR_INVALID_ARG
    assert call(wsp=ctypes.c_void_p(0x1010)) == ops.QMOE_ERR_INVALID_ARG  # not 256-aligned
    assert call(E=2000, wsb=1 << 30) == ops.QMOE_ERR_UNSUPPORTED
    assert ok


def test_align_noalloc_validation():
    """The no-allocation align refuses bad arguments like qmoe_align, and
    sizes whose workspace exceeds its static array, before touching the
    GPU."""
    L = ops.lib()
    p = ctypes.c_void_p(0x1000)
    lim = 1 << 20
    assert L.qmoe_align_noalloc(p, 64, 2, 8, 24, p, p, p, p, None, None) == \
        ops.QMOE_ERR_INVALID_ARG
    assert L.qmoe_align_noalloc(p, 64, 9, 8, 16, p, p, p, p, None, None) == \
        ops.QMOE_ERR_INVALID_ARG
    assert L.qmoe_align_noalloc(None, 64, 2, 8, 16, p, p, p, p, None, None) == \
        ops.QMOE_ERR_INVALID_ARG
    assert L.qmoe_align_noalloc(p, 64, 2, 8, 16, None, p, p, p, None, None) == \
        ops.QMOE_ERR_INVALID_ARG
    assert L.qmoe_align_noalloc(p, 64, 2, 2000, 16, p, p, p, p, None, None) == \
        ops.QMOE_ERR_UNSUPPORTED
    # the limit is the workspace qmoe_align would need
    assert L.qmoe_align_workspace(65024, 10, 1024) <= lim
    big = (65025, 10, 1024)
    assert L.qmoe_align_workspace(*big) > lim
    assert L.qmoe_align_noalloc(p, big[0], big[1], big[2], 16, p, p, p, p, None, None) == \
        ops.QMOE_ERR_UNSUPPORTED


def _desc(**kw):
    base = dict(scheme="a8w4", T=64, H=512, I=256, E=8, k=2, block_m=32, flags=0)
    base.update(kw)
    return ops.make_desc(base["scheme"], base["T"], base["H"], base["I"], base["E"], base["k"],
                         base["block_m"], base["flags"])


def test_ffn_workspace_and_desc_validation():
    L = ops.lib()
    ok = _desc()
    n = ops.grouped_ffn_workspace(ok)
    assert n > 0 and n % 256 == 0
    assert ops.grouped_ffn_workspace(_desc(T=128)) > n
    # dump flag adds the two int32 accumulator areas (w8a8 only)
    w8 = _desc(scheme="w8a8", I=128)
    w8d = _desc(scheme="w8a8", I=128, flags=ops.QMOE_FLAG_DUMP_ACC)
    assert ops.grouped_ffn_workspace(w8d) > ops.grouped_ffn_workspace(w8)
    a1, a2 = ops.grouped_ffn_debug_offsets(w8d)
    assert 0 < a1 < a2 < ops.grouped_ffn_workspace(w8d)
    for bad in (_desc(H=100), _desc(I=48), _desc(k=9), _desc(block_m=48), _desc(T=-1),
                _desc(scheme="w4a16", flags=8)):
        assert ops.grouped_ffn_workspace(bad) == 0
    p = ctypes.c_void_p(0x1000)
    w = ops.Weights(p, p, p, p)
    call = lambda d, ws=1 << 40, xs=p: L.qmoe_grouped_ffn(ctypes.byref(d), p, xs, ctypes.byref(w),
                                                           p, p, p, p, p, ws, None)
    assert call(_desc(H=100)) == ops.QMOE_ERR_INVALID_ARG
    assert call(_desc(H=288)) == ops.QMOE_ERR_UNSUPPORTED
    assert call(_desc(I=128)) == ops.QMOE_ERR_UNSUPPORTED  # a8w4 needs I % 256
    assert call(_desc(E=2000, k=2)) == ops.QMOE_ERR_UNSUPPORTED
    assert call(_desc(), ws=n - 1) == ops.QMOE_ERR_INVALID_ARG
    assert call(_desc(), xs=None) == ops.QMOE_ERR_INVALID_ARG  # a8w4 needs x_scale
    assert call(_desc(T=0)) == ops.QMOE_OK
    # 32-bit offsets inside the kernels: x (T*H), the stage-2 activations and
    # one expert's weights must each stay below 4 GiB.
    assert call(_desc(scheme="w4a16", T=1 << 19, H=4096, I=128)) == ops.QMOE_ERR_UNSUPPORTED
    assert call(_desc(scheme="w8a8", T=64, H=65536, I=65536)) == ops.QMOE_ERR_UNSUPPORTED
    assert L.qmoe_grouped_ffn(None, p, p, ctypes.byref(w), p, p, p, p, p, 1 << 40, None) == \
        ops.QMOE_ERR_INVALID_ARG
    # W4A8: scheme code 3; its scales are read 8 bytes at a time
    w4 = _desc(scheme="w4a8", I=128)
    w4d = _desc(scheme="w4a8", I=128, flags=ops.QMOE_FLAG_DUMP_ACC)
    assert ops.grouped_ffn_workspace(w4d) > ops.grouped_ffn_workspace(w4) > 0
    assert 0 < ops.grouped_ffn_debug_offsets(w4d)[0]
    w_mis = ops.Weights(p, ctypes.c_void_p(0x1004), p, p)
    assert L.qmoe_grouped_ffn(ctypes.byref(w4), p, p, ctypes.byref(w_mis), p, p, p, p, p,
                              1 << 40, None) == ops.QMOE_ERR_INVALID_ARG
    assert call(w4, xs=None) == ops.QMOE_ERR_INVALID_ARG  # w4a8 needs x_scale
    bad_scheme = ops.FfnDesc(4, 64, 512, 256, 8, 2, 32, 0)
    assert ops.grouped_ffn_workspace(bad_scheme) == 0
    assert call(bad_scheme) == ops.QMOE_ERR_INVALID_ARG


def test_decode_workspace_and_validation(monkeypatch):
    """qmoe_decode: the workspace does not depend on T (one zeroed workspace
    serves every batch size of a layer); every bad argument is refused before
    anything is launched."""
    L = ops.lib()
    INV, UNS = ops.QMOE_ERR_INVALID_ARG, ops.QMOE_ERR_UNSUPPORTED
    ws_of = lambda d: L.qmoe_decode_workspace(ctypes.byref(d))
    n = ws_of(_desc(T=1))
    assert n > 0 and n % 256 == 0
    assert ws_of(_desc(T=16)) == n == ws_of(_desc(T=5, block_m=48))  # block_m is not used
    assert ws_of(_desc(T=1, k=4)) > n
    for bad in (_desc(T=17), _desc(k=17, E=32), _desc(flags=ops.QMOE_FLAG_DUMP_ACC),
                _desc(T=-1), _desc(H=100), ops.FfnDesc(4, 1, 512, 256, 8, 2, 16, 0)):
        assert ws_of(bad) == 0
    p = ctypes.c_void_p(0x1000)
    w = ops.Weights(p, p, p, p)

    def call(d, ws=1 << 40, xs=p, logits=p, ob=p, of=None, wsp=p, w=w):
        return L.qmoe_decode(ctypes.byref(d), logits, p, xs, ctypes.byref(w), p, p, None, ob, of,
                             wsp, ws, None)

    assert call(_desc(T=0)) == ops.QMOE_OK
    assert call(_desc(T=17)) == UNS
    assert call(_desc(T=1, E=2000)) == UNS
    assert call(_desc(T=1, H=288)) == UNS
    assert call(_desc(T=1, I=128)) == UNS  # a8w4 needs I % 256
    assert call(_desc(T=1, I=4352)) == UNS  # quantized activations: I above 4096
    assert ws_of(_desc(T=1, I=4352)) == 0
    assert call(_desc(T=1, k=17, E=32)) == INV
    assert call(_desc(T=1, flags=ops.QMOE_FLAG_DUMP_ACC)) == INV
    assert call(_desc(T=1), logits=None) == INV
    assert call(_desc(T=1), ob=None, of=None) == INV
    assert call(_desc(T=1), xs=None) == INV  # a8w4 needs x_scale
    assert call(_desc(T=1), ws=n - 1) == INV
    assert call(_desc(T=1), wsp=ctypes.c_void_p(0x1010)) == INV  # 256-byte alignment
    w_mis = ops.Weights(p, ctypes.c_void_p(0x1004), p, p)
    assert call(_desc(T=1, scheme="w4a8", I=128), w=w_mis) == INV  # 8-byte w4a8 scales
    assert L.qmoe_decode(None, p, p, p, ctypes.byref(w), p, p, None, p, None, p, 1 << 40,
                         None) == INV
    monkeypatch.setenv("QMOE_DECODE_RING", "5")
    assert call(_desc(T=1)) == INV
    monkeypatch.delenv("QMOE_DECODE_RING")
    monkeypatch.setenv("QMOE_DECODE_G", "3")
    assert call(_desc(T=1)) == INV
    monkeypatch.setenv("QMOE_DECODE_G", "8")  # H 512: 16 chunks, not a multiple of 32
    assert call(_desc(T=1)) == INV


def test_combine_validation():
    L = ops.lib()
    p = ctypes.c_void_p(0x1000)
    assert L.qmoe_combine(p, 0, p, 4, 2, 12, p, None, None) == ops.QMOE_ERR_INVALID_ARG  # H % 8
    assert L.qmoe_combine(p, 7, p, 4, 2, 16, p, None, None) == ops.QMOE_ERR_INVALID_ARG  # dtype
    assert L.qmoe_combine(p, 0, p, 4, 2, 16, None, None, None) == ops.QMOE_ERR_INVALID_ARG
    assert L.qmoe_combine(None, 0, None, 0, 2, 16, p, None, None) == ops.QMOE_OK  # T = 0
    # T = 0 with empty (null) outputs as well: still a no-op, not an error.
    assert L.qmoe_combine(None, 0, None, 0, 2, 16, None, None, None) == ops.QMOE_OK


def test_prepack_validation():
    """Every bad argument of qmoe_prepack is refused on the host."""
    L = ops.lib()
    a, b, c, d = (ctypes.c_void_p(x) for x in (0x100000, 0x200000, 0x10000000, 0x20000000))
    INV = ops.QMOE_ERR_INVALID_ARG
    assert L.qmoe_prepack(4, 2, 32, 256, a, b, c, d, None) == INV          # scheme
    assert L.qmoe_prepack(-1, 2, 32, 256, a, b, c, d, None) == INV         # scheme
    assert L.qmoe_prepack(3, 2, 32, 64, a, b, c, d, None) == INV           # w4a8 K % 128
    assert L.qmoe_prepack(3, 2, 32, 256, a, b, c, None, None) == INV       # w4a8 needs scales_out
    assert L.qmoe_prepack(2, 0, 32, 256, a, b, c, d, None) == INV          # E
    assert L.qmoe_prepack(2, 2, 24, 256, a, b, c, d, None) == INV          # N % 16
    assert L.qmoe_prepack(2, 2, 32, 128, a, b, c, d, None) == INV          # a8w4 K % 256
    assert L.qmoe_prepack(0, 2, 32, 64, a, b, c, d, None) == INV           # K % 128
    assert L.qmoe_prepack(2, 2, 32, 256, None, b, c, d, None) == INV       # null codes
    assert L.qmoe_prepack(2, 2, 32, 256, a, b, None, d, None) == INV       # null output
    assert L.qmoe_prepack(2, 2, 32, 256, a, b, c, None, None) == INV       # a8w4 needs scales_out
    assert L.qmoe_prepack(2, 2, 32, 256, a, b, ctypes.c_void_p(0x100010), d, None) == INV  # overlap
    assert L.qmoe_prepack(2, 2, 32, 256, ctypes.c_void_p(0x100008), b, c, d, None) == INV  # align


def test_default_block_m_query():
    """qmoe_default_block_m: the tile table's row where there is one, else
    the rule on mean rows per expert; 0 for invalid arguments."""
    L = ops.lib()
    q = L.qmoe_default_block_m
    # rule (shapes without a table row): mean rows per expert = T*k/E
    assert q(2, 1, 2048, 1024, 500, 10) == 16        # 0.02 rows
    assert q(2, 1000, 2048, 1024, 500, 10) == 64     # 20 rows
    assert q(1, 2048, 2048, 768, 130, 8) == 64       # 126 rows, not a8w4
    assert q(2, 4000, 2048, 1024, 500, 10) == 128    # 80 rows
    assert q(2, 8000, 2048, 1024, 500, 10) == 128    # 160 rows, a8w4, inter 1024
    assert q(2, 8000, 2048, 512, 500, 10) == 64      # 160 rows, a8w4 share
    assert q(0, 8000, 2048, 1024, 500, 10) == 64     # 160 rows, not a8w4
    # table rows: the skewed long prefill keeps 128-row tiles for its heavy
    # experts, although its mean (160 rows) alone would give 64
    assert q(0, 8192, 4096, 1024, 512, 10) == 128
    for bad in ((4, 16, 256, 128, 8, 2), (0, -1, 256, 128, 8, 2), (0, 16, 256, 128, 8, 9),
                (0, 16, 0, 128, 8, 2)):
        assert q(*bad) == 0
