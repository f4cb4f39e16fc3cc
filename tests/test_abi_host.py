"""The C ABI library on a host without a GPU: it loads, exports every function
include/vsa.h declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from video_dit_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "vsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(vsa_\w+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared_functions()
    assert len(declared) >= 11, declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(_lib.SIGNATURES), "binding and header disagree"


def test_abi_version_and_status_strings():
    lib = _lib.load()
    assert lib.vsa_abi_version() == 6
    for s, name in [(0, "VSA_OK"), (1, "VSA_ERR_NULL"), (2, "VSA_ERR_SHAPE"),
                    (3, "VSA_ERR_UNSUPPORTED"), (4, "VSA_ERR_RANGE"), (5, "VSA_ERR_WORKSPACE"),
                    (6, "VSA_ERR_HIP")]:
        assert lib.vsa_status_string(s).decode() == name
    assert lib.vsa_status_string(99).decode() == "VSA_ERR_UNKNOWN"


def test_host_cube_functions():
    lib = _lib.load()
    assert lib.vsa_num_cubes(21, 30, 52) == 624
    assert lib.vsa_num_cubes(30, 48, 80) == 1920
    assert lib.vsa_num_cubes(0, 1, 1) == -1
    buf = (ctypes.c_int32 * 8)()
    assert lib.vsa_vbs_host(5, 6, 7, ctypes.cast(buf, ctypes.c_void_p), 8) == 0
    assert list(buf) == [64, 48, 32, 24, 16, 12, 8, 6]
    assert lib.vsa_vbs_host(5, 6, 7, ctypes.cast(buf, ctypes.c_void_p), 7) == _lib.VSA_ERR_SHAPE
    assert lib.vsa_vbs_host(5, 6, 7, None, 8) == _lib.VSA_ERR_NULL


# Fake, never-dereferenced but 256-byte aligned "device" addresses: every call
# below fails validation on the host before any HIP call is made.
P = 1 << 20


def test_tile_validation():
    lib = _lib.load()
    assert lib.vsa_tile(None, P, None, 1, 5, 6, 7, 2, 64, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_tile(P, P, None, 1, 0, 6, 7, 2, 64, None) == _lib.VSA_ERR_SHAPE
    assert lib.vsa_tile(P, P, None, 0, 5, 6, 7, 2, 64, None) == _lib.VSA_ERR_SHAPE
    assert lib.vsa_tile(P, P, None, 1, 5, 6, 7, 2, 96, None) == _lib.VSA_ERR_UNSUPPORTED
    assert lib.vsa_tile(P + 8, P, None, 1, 5, 6, 7, 2, 64, None) == _lib.VSA_ERR_UNSUPPORTED
    lib.vsa_tile(P, P, None, 1, 5, 6, 7, 2, 96, None)
    assert b"D=96" in lib.vsa_last_error()
    assert lib.vsa_untile(P, None, 1, 5, 6, 7, 2, 64, None) == _lib.VSA_ERR_NULL


def test_select_validation():
    lib = _lib.load()
    need = lib.vsa_select_workspace_bytes(1, 2, 8, 64)
    assert need >= 2 * 1 * 2 * 8 * 64 * 4 + 1 * 2 * 8 * 8 * 4
    assert lib.vsa_select_workspace_bytes(0, 2, 8, 64) == 0
    args = lambda topk, ws, wsb, nc=8, d=64: (P, P, P, 1, nc, 2, d, topk, P, ws, wsb, None)
    assert lib.vsa_select(*args(3, P, need)[:2], None, *args(3, P, need)[3:]) == _lib.VSA_ERR_NULL
    assert lib.vsa_select(*args(0, P, need)) == _lib.VSA_ERR_RANGE
    assert lib.vsa_select(*args(9, P, need)) == _lib.VSA_ERR_RANGE
    assert lib.vsa_select(*args(3, P, need - 1)) == _lib.VSA_ERR_WORKSPACE
    assert lib.vsa_select(*args(3, None, need)) == _lib.VSA_ERR_WORKSPACE
    assert lib.vsa_select(*args(3, P + 16, need)) == _lib.VSA_ERR_WORKSPACE
    assert lib.vsa_select(*args(3, P, need, nc=8193)) == _lib.VSA_ERR_UNSUPPORTED
    assert lib.vsa_select(*args(3, P, need, d=32)) == _lib.VSA_ERR_UNSUPPORTED


def test_fwd_validation():
    lib = _lib.load()

    def call(**kw):
        need = lib.vsa_fwd_workspace_bytes(1, 8, 8, 2, 64, 3)
        a = dict(q=P, k=P, v=P, idx=P, vbs=P, out=P, B=1, Nq=8, Nkv=8, NH=2, D=64, topk=3,
                 scale=0.0, ws=P, wsb=need)
        a.update(kw)
        return lib.vsa_fwd(a["q"], a["k"], a["v"], a["idx"], a["vbs"], a["out"], a["B"], a["Nq"],
                           a["Nkv"], a["NH"], a["D"], a["topk"], a["scale"], a["ws"], a["wsb"],
                           None)

    assert call(q=None) == _lib.VSA_ERR_NULL
    assert call(vbs=None) == _lib.VSA_ERR_NULL
    assert call(Nq=0) == _lib.VSA_ERR_SHAPE
    assert call(NH=-1) == _lib.VSA_ERR_SHAPE
    assert call(D=80) == _lib.VSA_ERR_UNSUPPORTED
    assert call(topk=0) == _lib.VSA_ERR_RANGE
    assert call(topk=9) == _lib.VSA_ERR_RANGE
    assert call(scale=float("nan")) == _lib.VSA_ERR_RANGE
    assert call(out=P + 2) == _lib.VSA_ERR_UNSUPPORTED
    # fp16 v (8 cubes x 64 rows x 2 heads x 64 x 2 bytes), then the tile
    # lists of the 16 (head, query cube) units ((2 * 3 + 4) tiles x 8 bytes
    # each = 1280 bytes), then their first and end tiles (16 x 2 int32 -> 256
    # after 256-byte rounding), the cube at each dispatch position and each
    # cube's position (16 int32 -> 256 each) and the positions' sort keys
    # (16 x 2 int32 -> 256), then the largest |v| of every (v pre-pass
    # workgroup, head) (8 cubes x 8 workgroups x 2 heads float32 = 512) and
    # the per-head exponent of the fp16 copy (2 int32 -> 256)
    need = 8 * 64 * 2 * 64 * 2 + 1280 + 256 + 256 + 256 + 256 + 512 + 256
    assert lib.vsa_fwd_workspace_bytes(1, 8, 8, 2, 64, 3) == need
    assert lib.vsa_fwd_workspace_bytes(1, 8, 8, 2, 64, 0) == 0
    assert call(ws=None) == _lib.VSA_ERR_WORKSPACE
    assert call(wsb=need - 1) == _lib.VSA_ERR_WORKSPACE
    # one batch of k must span < 4 GiB: Nkv * 64 * NH * D * 2 = Nkv * 16384 here
    assert call(Nkv=1 << 18, topk=3) == _lib.VSA_ERR_UNSUPPORTED
    assert call(ws=P + 128) == _lib.VSA_ERR_WORKSPACE


def test_fwd_splits_choice_and_workspace():
    """The key-range split count: none at the Wan shape (a head's K and fp16 V
    copy, 624 x 64 x 128 x 4 bytes = 20 MB, stay under 32 MiB), 2 at the 720p
    shape (1920 cubes: 63 MB in splits of about 32 MiB), 4 at 4,096 cubes, at
    most topk / 8, never for rows longer than 1024 ids; forced counts are
    taken as given. With splits the workspace adds the partial results."""
    lib = _lib.load()
    assert lib.vsa_fwd_splits(624, 128, 78, 0) == 1
    assert lib.vsa_fwd_splits(1920, 128, 192, 0) == 2
    assert lib.vsa_fwd_splits(4096, 128, 192, 0) == 4
    assert lib.vsa_fwd_splits(4096, 128, 24, 0) == 3
    assert lib.vsa_fwd_splits(1920, 128, 8, 0) == 1
    assert lib.vsa_fwd_splits(1920, 128, 1100, 0) == 1
    assert lib.vsa_fwd_splits(1920, 128, 1100, 4) == 1
    assert lib.vsa_fwd_splits(1920, 128, 192, 1) == 1
    assert lib.vsa_fwd_splits(8, 64, 3, 3) == 3
    assert lib.vsa_fwd_splits(8, 64, 3, 16) == 16
    assert lib.vsa_fwd_splits(8, 64, 3, 17) == 0
    assert lib.vsa_fwd_splits(8, 64, 9, 0) == 0
    # 3 splits of 16 units: lists of 2 * 3 + 4 + 3 * 5 tiles (a zero quarter
    # and 4 zero tiles per split) x 8 bytes = 3200 -> 3328, first tiles
    # (16 x 4 int32 = 256), order, positions and keys (256 + 256 + 256), |v|
    # maxima (512), exponents (256), partial O (16 x 3 x 64 x 64 float32) and
    # partial row states (16 x 3 x 64 float4)
    need = 8 * 64 * 2 * 64 * 2 + 3328 + 256 + 256 + 256 + 256 + 512 + 256 + \
        16 * 3 * 64 * 64 * 4 + 16 * 3 * 64 * 16
    assert lib.vsa_fwd_workspace_bytes_ex(1, 8, 8, 2, 64, 3, 3) == need
    assert lib.vsa_fwd_workspace_bytes_ex(1, 8, 8, 2, 64, 3, 0) == \
        lib.vsa_fwd_workspace_bytes(1, 8, 8, 2, 64, 3)
    assert lib.vsa_fwd_workspace_bytes_ex(1, 8, 8, 2, 64, 3, 17) == 0

    def lut(splits, wsb=need):
        return lib.vsa_fwd_lut_ex(P, P, P, P, None, P, P, None, None, 1, 8, 8, 2, 64, 3, 0.0,
                                  splits, P, wsb, None)

    assert lut(-1) == _lib.VSA_ERR_RANGE
    assert lut(17) == _lib.VSA_ERR_RANGE
    assert lut(3, need - 1) == _lib.VSA_ERR_WORKSPACE


def test_select_noalloc_validation():
    """The allocation-free selector rejects bad arguments on the host, and a
    shape whose single head needs more than its static scratch."""
    lib = _lib.load()
    cap = lib.vsa_select_noalloc_max_bytes()
    assert cap == 64 << 20
    args = lambda topk, nc=8, d=64, q=P: (q, P, P, 1, nc, 2, d, topk, P, None)
    assert lib.vsa_select_noalloc(*args(3, q=None)) == _lib.VSA_ERR_NULL
    assert lib.vsa_select_noalloc(*args(0)) == _lib.VSA_ERR_RANGE
    assert lib.vsa_select_noalloc(*args(9)) == _lib.VSA_ERR_RANGE
    assert lib.vsa_select_noalloc(*args(3, d=80)) == _lib.VSA_ERR_UNSUPPORTED
    assert lib.vsa_select_noalloc(*args(3, nc=8193)) == _lib.VSA_ERR_UNSUPPORTED
    # one head of 4096 cubes at D = 128: 4096^2 x 4 bytes of scores alone
    assert lib.vsa_select_workspace_bytes(1, 1, 4096, 128) > cap
    assert lib.vsa_select_noalloc(*args(4, nc=4096, d=128)) == _lib.VSA_ERR_UNSUPPORTED
    assert b"scratch" in lib.vsa_last_error()


def test_coarse_and_combine_validation():
    lib = _lib.load()
    sel = lib.vsa_select_workspace_bytes(1, 2, 8, 64)
    need = lib.vsa_coarse_workspace_bytes(1, 2, 8, 64)
    assert need == sel + 1 * 2 * 8 * 64 * 4          # + pooled v, a multiple of 256
    assert lib.vsa_coarse_workspace_bytes(1, 2, 0, 64) == 0

    def coarse(**kw):
        a = dict(q=P, k=P, v=P, vbs=P, B=1, Nc=8, NH=2, D=64, topk=3, idx=P, scale=0.0, oc=P,
                 ws=P, wsb=need)
        a.update(kw)
        return lib.vsa_coarse(a["q"], a["k"], a["v"], a["vbs"], a["B"], a["Nc"], a["NH"], a["D"],
                              a["topk"], a["idx"], a["scale"], a["oc"], a["ws"], a["wsb"], None)

    assert coarse(v=None) == _lib.VSA_ERR_NULL
    assert coarse(oc=None) == _lib.VSA_ERR_NULL
    assert coarse(Nc=0) == _lib.VSA_ERR_SHAPE
    assert coarse(D=96) == _lib.VSA_ERR_UNSUPPORTED
    assert coarse(Nc=8193) == _lib.VSA_ERR_UNSUPPORTED
    assert coarse(topk=0) == _lib.VSA_ERR_RANGE
    assert coarse(topk=9) == _lib.VSA_ERR_RANGE
    assert coarse(scale=float("inf")) == _lib.VSA_ERR_RANGE
    assert coarse(oc=P + 4) == _lib.VSA_ERR_UNSUPPORTED
    assert coarse(wsb=need - 1) == _lib.VSA_ERR_WORKSPACE
    assert coarse(ws=P + 64) == _lib.VSA_ERR_WORKSPACE

    def comb(**kw):
        a = dict(of=P, oc=P, gc=P, gf=P, out=P, B=1, Nc=8, NH=2, D=64)
        a.update(kw)
        return lib.vsa_gate_combine(a["of"], a["oc"], a["gc"], a["gf"], a["out"], a["B"], a["Nc"],
                                    a["NH"], a["D"], None)

    assert comb(gf=None) == _lib.VSA_ERR_NULL
    assert comb(Nc=-1) == _lib.VSA_ERR_SHAPE
    assert comb(D=32) == _lib.VSA_ERR_UNSUPPORTED
    assert comb(out=P + 8) == _lib.VSA_ERR_UNSUPPORTED
    assert comb(Nc=1 << 26) == _lib.VSA_ERR_SHAPE      # more token rows than grid slots


@pytest.mark.parametrize("grid", [(21, 30, 52), (30, 48, 80), (5, 6, 7), (1, 1, 1), (17, 3, 90),
                                  (64, 4, 4)])
def test_cube_order_host_matches_oracle(grid):
    import numpy as np

    import oracle
    lib = _lib.load()
    n = lib.vsa_num_cubes(*grid)
    for kind, name in ((_lib.VSA_ORDER_HILBERT, "hilbert"), (_lib.VSA_ORDER_ROW_MAJOR, "row_major")):
        buf = (ctypes.c_int32 * n)()
        assert lib.vsa_cube_order_host(*grid, kind, buf, n) == _lib.VSA_OK
        assert np.array_equal(np.frombuffer(buf, dtype=np.int32), oracle.cube_order(*grid, name))


def test_order_and_mask_validation():
    lib = _lib.load()
    buf = (ctypes.c_int32 * 8)()
    assert lib.vsa_cube_order_host(5, 6, 7, 1, None, 8) == _lib.VSA_ERR_NULL
    assert lib.vsa_cube_order_host(5, 6, 7, 1, buf, 7) == _lib.VSA_ERR_SHAPE
    assert lib.vsa_cube_order_host(5, 6, 7, 2, buf, 8) == _lib.VSA_ERR_RANGE
    assert lib.vsa_cube_order_host(0, 6, 7, 1, buf, 8) == _lib.VSA_ERR_SHAPE
    assert lib.vsa_tile_ordered(P, P, None, None, 1, 5, 6, 7, 2, 64, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_tile_ordered(P, P, None, P, 1, 5, 6, 7, 2, 96, None) == _lib.VSA_ERR_UNSUPPORTED
    assert lib.vsa_untile_ordered(P, P, None, 1, 5, 6, 7, 2, 64, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_untile_ordered(P, P + 4, P, 1, 5, 6, 7, 2, 64, None) == _lib.VSA_ERR_UNSUPPORTED
    m = lambda **kw: lib.vsa_mask_to_lut(*[kw.get(k, d) for k, d in (
        ("mask", P), ("B", 1), ("NH", 2), ("Nq", 8), ("Nkv", 8), ("max_kv", 8), ("idx", P),
        ("cnt", P), ("tr", None))], None)
    assert m(mask=None) == _lib.VSA_ERR_NULL
    assert m(cnt=None) == _lib.VSA_ERR_NULL
    assert m(Nq=0) == _lib.VSA_ERR_SHAPE
    assert m(max_kv=0) == _lib.VSA_ERR_RANGE
    assert m(max_kv=9) == _lib.VSA_ERR_RANGE
    assert m(B=65536, NH=65536, Nq=2) == _lib.VSA_ERR_SHAPE


def test_validate_topk_validation():
    lib = _lib.load()
    assert lib.vsa_validate_topk(None, 1, 1, 8, 8, 3, P, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_validate_topk(P, 1, 1, 8, 0, 3, P, None) == _lib.VSA_ERR_SHAPE
    assert lib.vsa_validate_topk(P, 1, 1, 8, 9000, 3, P, None) == _lib.VSA_ERR_UNSUPPORTED
    assert lib.vsa_validate_topk(P, 1, 1, 8, 8, 0, P, None) == _lib.VSA_ERR_RANGE


def test_python_binding_rejects_cpu_tensors():
    import torch

    import video_dit_block_amd as vsa
    x = torch.zeros(1, 210, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        vsa.tile(x, 5, 6, 7)
