"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every function include/*.h declares, and rejects bad arguments before it
touches the device."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(cco_\w+)\s*\(", src, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def capi():
    from combine_symmetric_memory_amd import _capi
    return _capi


def test_header_declares_the_path_entry_points():
    names = _declared_functions()
    for n in ("cco_sym_heap_create", "cco_moe_plan", "cco_moe_dispatch", "cco_moe_expert",
              "cco_moe_combine"):
        assert n in names


def test_library_exports_every_declared_symbol(capi):
    names = _declared_functions()
    assert len(names) >= 15
    bound = {s[0] for s in capi.SIGNATURES}
    for n in sorted(names):
        assert hasattr(capi.lib, n), "missing export " + n
        assert n in bound, "binding does not declare " + n


def test_status_strings(capi):
    assert capi.status_string(0) == "CCO_OK"
    assert capi.status_string(-5) == "CCO_ERR_BAD_EXPERT"
    assert capi.status_string(-4) == "CCO_ERR_CAPACITY"


def _shape(capi, T=128, H=256, K=2, E=8, I=512):
    return capi.cco_moe_shape(T, H, K, E, I)


def test_required_bytes_and_layout(capi):
    s = _shape(capi)
    n = capi.lib.cco_moe_required_slot_bytes(ctypes.byref(s), 4)
    lay = capi.cco_moe_layout()
    assert capi.lib.cco_moe_layout_of(ctypes.byref(s), 4, ctypes.byref(lay)) == 0
    cap = 128 * min(2, 8 // 4)
    assert lay.cap == cap
    assert lay.disp_x_bytes == cap * 256 * 2
    assert lay.disp_meta_bytes == cap * 12
    assert lay.hbuf_bytes == cap * 512 * 2
    assert lay.out_tok_bytes == cap * 256 * 2
    offs = [lay.disp_x, lay.disp_meta, lay.hbuf, lay.out_tok]
    sizes = [lay.disp_x_bytes, lay.disp_meta_bytes, lay.hbuf_bytes, lay.out_tok_bytes]
    for o in offs:
        assert o % 4096 == 0
    # windows do not overlap and leave room for the guard bytes
    for i in range(3):
        assert offs[i] + sizes[i] + 256 <= offs[i + 1]
    assert n >= offs[-1] + sizes[-1] + 256
    # identity experts: no HBUF / OUT_TOK
    s0 = _shape(capi, I=0)
    assert capi.lib.cco_moe_layout_of(ctypes.byref(s0), 4, ctypes.byref(lay)) == 0
    assert lay.hbuf_bytes == 0 and lay.out_tok_bytes == 0


@pytest.mark.parametrize("kw,nslots", [
    (dict(H=250), 4),             # H % 8
    (dict(E=6), 4),               # E % S
    (dict(K=0), 4),
    (dict(K=33), 4),              # K above the limit
    (dict(E=2048), 4),            # E above the limit
    (dict(I=100), 4),             # I % 128
    (dict(I=192), 4),             # I % 128
    (dict(H=264, I=512), 4),      # H % 256 with SwiGLU experts
    (dict(H=384, I=512), 4),      # H % 256 with SwiGLU experts
    (dict(H=16384, I=32768), 4),  # one expert's gate+up weights reach 2 GiB
    (dict(T=-1), 4),
    (dict(), 0),
])
def test_invalid_shapes_rejected(capi, kw, nslots):
    s = _shape(capi, **kw)
    assert capi.lib.cco_moe_required_slot_bytes(ctypes.byref(s), nslots) == 0
    lay = capi.cco_moe_layout()
    assert capi.lib.cco_moe_layout_of(ctypes.byref(s), nslots, ctypes.byref(lay)) == -1


def test_invalid_calls_rejected_before_the_device(capi):
    L = capi.lib
    h = ctypes.c_void_p()
    assert L.cco_sym_heap_create(0, 0, 1 << 20, ctypes.byref(h)) == -1
    assert L.cco_sym_heap_create(0, 4, 0, ctypes.byref(h)) == -1
    assert L.cco_sym_heap_create(-1, 4, 1 << 20, ctypes.byref(h)) == -1
    assert L.cco_sym_heap_create(0, 4, 1 << 20, None) == -1
    assert L.cco_sym_heap_destroy(None) == 0
    assert L.cco_sym_heap_slot_ptr(None, 0, 0) is None
    assert L.cco_moe_create(None, None, None) == -1
    assert L.cco_moe_plan(None, None, 0, None) == -1
    assert L.cco_moe_dispatch(None, None, None, 0, None) == -1
    assert L.cco_moe_dispatch_fp8(None, None, None, 0, None, 0, None) == -1
    assert L.cco_moe_expert(None, None, None, None) == -1
    assert L.cco_moe_combine(None, None, None, None, 0, None) == -1
    assert L.cco_moe_status(None, None, None, None) == -1
    assert L.cco_moe_dispatch_view(None, 0) is None
    assert L.cco_moe_combine_in_view(None, 0) is None
    assert L.cco_moe_set_timing(None, 1) == -1
    assert L.cco_moe_timing_summary(None, None, None) == -1
