"""The C-ABI library: it loads, exports every symbol include/*.h declares, and rejects bad
arguments on the host before launching anything (no GPU needed: no call below reaches
the device)."""
import ctypes
import os
import re

import pytest

import block_scaled_fp8_dispatch_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if not h.endswith(".h"):
            continue
        text = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libmoe.so is not built (run python -m block_scaled_fp8_dispatch_amd.build)")
    return moe.load_library()


def test_exports_every_declared_symbol(lib):
    declared = _header_functions()
    assert declared == set(moe.EXPORTED), declared ^ set(moe.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert moe.moe_version() >= 10000
    assert moe.moe_status_string(moe.MOE_OK) == "ok"
    assert "align" in moe.moe_status_string(moe.MOE_ERR_ALIGN)
    assert moe.moe_status_string(12345) == "unknown status"


def test_sizes_and_shape_validation(lib):
    good = moe.make_shape(8, 7168, 18432, 2, 8192)
    assert moe.moe_packed_weights_bytes(good) == 8 * (2 * 18432 * 7168 // 2 + 2 * 18432 * 7168 // 32
                                                      + 7168 * 18432 // 2 + 7168 * 18432 // 32)
    assert moe.moe_workspace_bytes(good) > 8192 * 2 * 7168 * 2
    for bad in (moe.make_shape(0, 256, 128, 1, 1), moe.make_shape(4, 200, 128, 1, 1),
                moe.make_shape(4, 256, 100, 1, 1), moe.make_shape(4, 256, 128, 5, 1),
                moe.make_shape(4, 256, 128, 0, 1), moe.make_shape(4, 256, 128, 1, -1),
                moe.make_shape(2000, 256, 128, 1, 1), moe.make_shape(4, 256, 128, 65, 100),
                moe.make_shape(4, 64, 128, 1, 1), moe.make_shape(4, 128, 0, 1, 1)):
        assert moe.moe_packed_weights_bytes(bad) == 0
        assert moe.moe_workspace_bytes(bad) == 0
    # H and I need only be multiples of 128; with H an odd multiple of 128, W2's last column
    # tile of 256 rows is completed with zero rows
    for E, H, I in ((4, 128, 128), (4, 384, 128), (3, 640, 384)):
        nb = moe.moe_packed_weights_bytes(moe.make_shape(E, H, I, 2, 64))
        h_pad = -(-H // 256) * 256
        w1 = E * (2 * I * H // 2 + I // 128 * (-(-H // 512)) * 16 * 64 * 4)
        w2 = E * (h_pad * I // 2 + h_pad // 256 * (-(-I // 512)) * 16 * 64 * 4)
        assert w1 + w2 <= nb < w1 + w2 + 4 * 256, (E, H, I)
        assert moe.moe_workspace_bytes(moe.make_shape(E, H, I, 2, 64)) > 0


def test_layout_is_consistent(lib):
    s = moe.make_shape(32, 7168, 2048, 8, 4096)
    L = moe.moe_workspace_layout(s, 4096)
    assert L["total"] == moe.moe_workspace_bytes(s)
    assert L["block_m"] == 256
    assert moe.moe_workspace_layout(s, 128)["block_m"] == 64
    offs = [L[k] for k in ("meta", "counts", "offsets", "perm", "inv", "tile_expert", "tile_row0",
                           "h8", "h_sf", "stage", "xg", "xg_sf")]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert L["h_sf_stride"] == 4 * ((2048 + 511) // 512)
    with pytest.raises(moe.MoEError):
        moe.moe_workspace_layout(s, 4097)


def test_dispatch_copy_region_only_for_small_topk(lib):
    # k = 8: Linear1 gathers x through perm, so the blocked copy of x takes no bytes; the
    # blocked copy of its scale rows is always there
    T, E, H = 4096, 32, 7168
    L8 = moe.moe_workspace_layout(moe.make_shape(E, H, 2048, 8, T), T)
    assert L8["xg"] == L8["xg_sf"]
    assert L8["total"] - L8["xg_sf"] >= (T * 8 + E * 255) * 4 * ((H + 511) // 512)
    # k = 2: one H-byte row and its scale words per padded row
    T, E, H = 4096, 8, 7168
    L2 = moe.moe_workspace_layout(moe.make_shape(E, H, 2048, 2, T), T)
    ppad = T * 2 + E * 255
    assert L2["xg_sf"] - L2["xg"] >= ppad * H
    assert L2["total"] - L2["xg_sf"] >= ppad * 4 * ((H + 511) // 512)


def test_forward_host_errors(lib):
    s = moe.make_shape(4, 256, 512, 2, 64)
    ws_bytes = moe.moe_workspace_bytes(s)
    A = 0x10000  # aligned fake addresses: every case below returns before touching them
    args = dict(y=A, x=A, xsf=A, idx=A, w=A, packed=A, ws=A)

    def call(T=64, shape=s, wsb=ws_bytes, **over):
        a = dict(args, **over)
        return moe.moe_forward_raw(a["y"], a["x"], a["xsf"], a["idx"], a["w"], T, shape,
                                   a["packed"], a["ws"], wsb, None)

    assert call(y=None) == moe.MOE_ERR_NULL
    assert call(idx=None) == moe.MOE_ERR_NULL
    assert call(ws=None) == moe.MOE_ERR_NULL
    assert call(x=A + 8) == moe.MOE_ERR_ALIGN
    assert call(w=A + 4) == moe.MOE_ERR_ALIGN
    assert call(wsb=ws_bytes - 1) == moe.MOE_ERR_WORKSPACE
    assert call(T=65) == moe.MOE_ERR_TOKENS
    assert call(T=-1) == moe.MOE_ERR_TOKENS
    assert call(shape=moe.make_shape(4, 250, 512, 2, 64)) == moe.MOE_ERR_SHAPE
    assert call(T=0) == moe.MOE_OK    # nothing to do: no launch


def test_prepare_host_errors(lib):
    s = moe.make_shape(4, 256, 512, 2, 64)
    nb = moe.moe_packed_weights_bytes(s)
    A = 0x10000
    assert moe.moe_prepare_weights_raw(s, None, A, A, A, A, nb, None) == moe.MOE_ERR_NULL
    assert moe.moe_prepare_weights_raw(s, A, A + 1, A, A, A, nb, None) == moe.MOE_ERR_ALIGN
    assert moe.moe_prepare_weights_raw(s, A, A, A, A, A, nb - 1, None) == moe.MOE_ERR_WORKSPACE
    bad = moe.make_shape(4, 256, 100, 2, 64)
    assert moe.moe_prepare_weights_raw(bad, A, A, A, A, A, nb, None) == moe.MOE_ERR_SHAPE


def test_missing_library_fails_loudly(tmp_path):
    from block_scaled_fp8_dispatch_amd import _lib
    saved = _lib._lib
    try:
        _lib._lib = None
        with pytest.raises(ImportError):
            _lib.load_library(str(tmp_path / "nope.so"))
    finally:
        _lib._lib = saved


def test_gemm_sizes_and_host_errors(lib):
    G, N, K = 4, 2112, 7168
    nb = moe.moe_gemm_packed_b_bytes(G, N, K)
    # N padded to 9 tiles of 256 rows: FP4 data + one 32-bit scale word per lane, fragment and 512 K
    assert nb == G * 9 * 256 * K // 2 + G * 9 * ((K + 511) // 512) * 16 * 64 * 4
    for bad in ((0, 256, 256), (1025, 256, 256), (1, 8, 256), (1, 264, 256), (1, 256, 64),
                (1, 256, 320)):
        assert moe.moe_gemm_packed_b_bytes(*bad) == 0
    assert moe.moe_gemm_workspace_bytes(-1, 1) == 0 and moe.moe_gemm_workspace_bytes(10, 0) == 0
    wsb = moe.moe_gemm_workspace_bytes(64, 1)
    A = 0x10000
    call = moe.gemm_call_raw
    P = lambda **o: dict(dict(d=A, a=A, asf=A, b=A, ws=A), **o)

    def dense(m=64, n=256, k=512, wb=wsb, **o):
        p = P(**o)
        return call("moe_fp8_fp4_gemm", p["d"], p["a"], p["asf"], m, n, k, p["b"], p["ws"], wb, None)

    assert dense(d=None) == moe.MOE_ERR_NULL
    assert dense(n=100) == moe.MOE_ERR_SHAPE
    assert dense(k=384 + 64) == moe.MOE_ERR_SHAPE
    assert dense(a=A + 4) == moe.MOE_ERR_ALIGN
    assert dense(m=-1) == moe.MOE_ERR_TOKENS
    assert dense(m=2 ** 24, k=512) == moe.MOE_ERR_TOKENS        # m * k >= 2^32
    assert dense(wb=wsb - 1) == moe.MOE_ERR_WORKSPACE
    assert dense(m=0) == moe.MOE_OK

    def contig(m=64, groups=3, wb=None, **o):
        p = P(**o)
        wb = moe.moe_gemm_workspace_bytes(m, groups) if wb is None else wb
        return call("moe_m_grouped_fp8_fp4_gemm_contiguous", p["d"], p["a"], p["asf"], A, m, groups,
                    256, 512, p["b"], p["ws"], wb, None)

    assert contig(groups=0, wb=1 << 20) == moe.MOE_ERR_SHAPE
    assert contig(ws=None) == moe.MOE_ERR_NULL
    assert contig(wb=moe.moe_gemm_workspace_bytes(64, 3) - 1) == moe.MOE_ERR_WORKSPACE
    assert contig(m=0) == moe.MOE_OK

    def masked(groups=3, max_m=16, wb=None, **o):
        p = P(**o)
        wb = moe.moe_gemm_workspace_bytes(max(groups * max_m, 0), max(groups, 1)) if wb is None else wb
        return call("moe_m_grouped_fp8_fp4_gemm_masked", p["d"], p["a"], p["asf"], A, groups, max_m, 8,
                    256, 512, p["b"], p["ws"], wb, None)

    assert masked(max_m=-1, wb=1 << 20) == moe.MOE_ERR_TOKENS
    assert masked(wb=moe.moe_gemm_workspace_bytes(48, 3) - 1) == moe.MOE_ERR_WORKSPACE
    assert masked(d=A + 2) == moe.MOE_ERR_ALIGN
    assert masked(max_m=0) == moe.MOE_OK

    assert call("moe_cast_to_fp8", A, 4, 200, A, A, None) == moe.MOE_ERR_SHAPE
    assert call("moe_cast_to_fp8", A, -1, 256, A, A, None) == moe.MOE_ERR_TOKENS
    assert call("moe_cast_to_fp8", None, 4, 256, A, A, None) == moe.MOE_ERR_NULL
    assert call("moe_cast_to_fp8", A, 4, 256, A + 8, A, None) == moe.MOE_ERR_ALIGN
    assert call("moe_cast_to_fp8", A, 0, 256, A, A, None) == moe.MOE_OK
    assert call("moe_gemm_prepare_b", 1, 256, 512, A, A, A, moe.moe_gemm_packed_b_bytes(1, 256, 512) - 1,
                None) == moe.MOE_ERR_WORKSPACE
