"""C ABI checks that need no GPU: the library loads, exports every symbol
declared in include/hyb.h, plans layouts identical to the oracle's, and
rejects bad arguments on the host before anything is enqueued (every call
below fails validation, so no HIP work is ever started)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from matmul_pack_b1_amd import binding as hb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hyb.h")


@pytest.fixture(scope="module")
def L():
    return hb.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hyb_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header(L):
    names = declared_functions()
    assert set(names) == set(hb.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", hb.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (hyb_\w+)", out))
    for name in names:
        assert name in exported, name
        assert getattr(L, name) is not None


def test_abi_version_and_status_strings(L):
    assert L.hyb_abi_version() == 1
    for code, name in enumerate(["HYB_OK", "HYB_ERR_INVALID_ARG", "HYB_ERR_SHAPE", "HYB_ERR_DTYPE",
                                 "HYB_ERR_UNSUPPORTED", "HYB_ERR_FORMAT", "HYB_ERR_HIP"]):
        assert hb.status_str(code) == name
    assert hb.status_str(99) == "HYB_ERR_UNKNOWN"


def test_layout_struct_size():
    assert ctypes.sizeof(hb.HybLayout) == 8 + 16 + 16 + 8 * 8
    assert ctypes.sizeof(hb.HybPacked) == 32


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("meta", ["idx2", "mask4", "mask8"])
def test_plan_matches_oracle(seed, meta):
    rng = np.random.default_rng(seed)
    b1 = int(rng.choice([64, 128, 256]))
    b2 = int(rng.choice([64, 128, 256]))
    tn, tk = int(rng.integers(0, 5)), int(rng.integers(0, 5))
    tmap = (rng.random((tn, tk)) < rng.random()).astype(np.uint8)
    lay, tidx = hb.plan(tn * b1, tk * b2, b1, b2, "bf16", meta, tmap)
    ref = oracle.plan(tn * b1, tk * b2, b1, b2, tmap)
    np.testing.assert_array_equal(tidx, ref["tidx"])
    assert lay.magic == hb.HYB_MAGIC and lay.version == hb.HYB_VERSION
    assert (lay.n_dense, lay.n_sparse) == (ref["n_dense"], ref["n_sparse"])
    for key in ("dense_bytes", "val_bytes", "meta_bytes", "tidx_bytes"):
        assert getattr(lay, key) == ref[key], key


def test_plan_8b_up_projection_sizes():
    from matmul_pack_b1_amd import workloads as wl
    mat = wl.workload(2).matrices[0]
    lay, _ = hb.plan(mat.n, mat.k, mat.b1, mat.b2, "bf16", "idx2", mat.tile_map())
    assert lay.dense_bytes + lay.val_bytes + lay.meta_bytes == 81_471_488


@pytest.mark.parametrize("args,code", [
    ((100, 128, 64, 64, "bf16", "idx2"), 2),    # n not a whole number of tiles
    ((128, 100, 64, 64, "bf16", "idx2"), 2),    # k not a whole number of tiles
    ((128, 128, 64, 48, "bf16", "idx2"), 2),    # b2 % 64 != 0
    ((128, 128, 8, 64, "bf16", "idx2"), 2),     # b1 % 16 != 0
    ((-64, 128, 64, 64, "bf16", "idx2"), 2),    # negative
    ((128, 128, 64, 64, "f32", "idx2"), 3),     # weight dtype
    ((128, 128, 64, 64, "bf16", "bits"), 1),    # metadata kind
])
def test_plan_rejects(args, code):
    n, k, b1, b2, dt, meta = args
    tm = np.zeros(4, np.uint8)
    with pytest.raises(hb.HybError) as e:
        hb.plan(n, k, b1, b2, dt, meta, tm)
    assert e.value.status == code
    assert hb.last_error()


def test_plan_rejects_map_values():
    with pytest.raises(hb.HybError) as e:
        hb.plan(128, 128, 64, 64, "bf16", "idx2", np.array([0, 1, 2, 0], np.uint8))
    assert e.value.status == 1 and "tile_map[2]" in hb.last_error()


def test_plan_null_map_and_out(L):
    lay = hb.HybLayout()
    assert L.hyb_plan(128, 128, 64, 64, 2, 1, None, ctypes.byref(lay), None) == 1
    assert L.hyb_plan(0, 128, 64, 64, 2, 1, None, ctypes.byref(lay), None) == 0  # no tiles: map unused
    assert L.hyb_plan(128, 128, 64, 64, 2, 1, None, None, None) == 1


def _good_layout(b1=128, b2=128, n=256, k=256):
    lay, tidx = hb.plan(n, k, b1, b2, "bf16", "idx2", np.array([[1, 0], [0, 1]], np.uint8)[: n // b1, : k // b2])
    return lay


FAKE = 0x10000  # a 16-byte aligned address; never dereferenced because validation fails first


def _call(L, fn, lay, packed=None, x=FAKE, m=1, ldx=256, y=FAKE, ydt=3, ldy=256):
    if packed is None:
        packed = hb.HybPacked(FAKE, FAKE, FAKE, FAKE)
    return getattr(L, fn)(ctypes.byref(lay) if lay is not None else None,
                          ctypes.byref(packed) if packed is not False else None,
                          x, m, ldx, y, ydt, ldy, None)


@pytest.mark.parametrize("fn", ["hyb_gemv", "hyb_gemm", "hyb_gemm_mfma", "hyb_gemm_noalloc"])
def test_product_rejects(L, fn):
    lay = _good_layout()
    assert _call(L, fn, None) == 1                          # null layout
    bad = hb.HybLayout.from_buffer_copy(lay)
    bad.magic = 0
    assert _call(L, fn, bad) == 5                           # magic
    bad = hb.HybLayout.from_buffer_copy(lay)
    bad.version = 2
    assert _call(L, fn, bad) == 5                           # version
    bad = hb.HybLayout.from_buffer_copy(lay)
    bad.val_bytes += 16
    assert _call(L, fn, bad) == 5                           # sizes
    bad = hb.HybLayout.from_buffer_copy(lay)
    bad.n_dense += 1
    assert _call(L, fn, bad) == 5                           # counts
    assert _call(L, fn, lay, m=-1) == 2                     # m < 0
    if fn == "hyb_gemv":
        assert _call(L, fn, lay, m=17) == 2                 # decode kernel m <= 16
    assert _call(L, fn, lay, ydt=1) == 3                    # fp16 out for bf16 weights
    assert _call(L, fn, lay, ydt=7) == 3
    assert _call(L, fn, lay, packed=False) == 1             # null descriptor
    assert _call(L, fn, lay, packed=hb.HybPacked(None, FAKE, FAKE, FAKE)) == 1
    assert _call(L, fn, lay, packed=hb.HybPacked(FAKE + 8, FAKE, FAKE, FAKE)) == 1
    assert _call(L, fn, lay, packed=hb.HybPacked(FAKE, FAKE, FAKE, None)) == 1
    assert _call(L, fn, lay, x=None) == 1                   # null x
    assert _call(L, fn, lay, x=FAKE + 2) == 1               # x alignment
    assert _call(L, fn, lay, ldx=255) == 1                  # ldx < k
    assert _call(L, fn, lay, ldx=260) == 1                  # ldx % 8
    assert _call(L, fn, lay, y=None) == 1                   # null y
    assert _call(L, fn, lay, ldy=100) == 1                  # ldy < n
    assert _call(L, fn, lay, y=FAKE + 2) == 1               # fp32 y alignment
    assert hb.last_error()


def _grouped(L, count, lays, packs=None, x=FAKE, m=1, ldx=256, ys=None, ydt=3, ldys=None):
    n = max(count, 1)
    la = (hb.HybLayout * n)(*lays) if lays is not None else None
    pk = (hb.HybPacked * n)(*(packs or [hb.HybPacked(FAKE, FAKE, FAKE, FAKE)] * len(lays or []))) \
        if lays is not None else None
    ya = (ctypes.c_void_p * n)(*(ys or [FAKE] * n))
    la_y = (ctypes.c_int64 * n)(*(ldys or [256] * n))
    return L.hyb_gemv_grouped(count, la, pk, x, m, ldx, ya, ydt, la_y, None)


def test_gemv_grouped_rejects(L):
    lay = _good_layout()
    assert _grouped(L, 0, None) == 0                               # count 0: no-op, arrays unused
    assert _grouped(L, -1, [lay]) == 2                             # count < 0
    assert _grouped(L, hb.MAX_GROUP + 1, [lay] * (hb.MAX_GROUP + 1)) == 2
    assert L.hyb_gemv_grouped(1, None, None, FAKE, 1, 256, None, 3, None, None) == 1
    assert _grouped(L, 2, [lay, lay], m=17) == 2                   # decode kernel m <= 16
    bad = hb.HybLayout.from_buffer_copy(lay)
    bad.magic = 0
    assert _grouped(L, 2, [lay, bad]) == 5
    assert "matrix 1" in hb.last_error()
    other_k = _good_layout(k=128, b2=128, n=256)                   # k = 128 instead of 256
    assert _grouped(L, 2, [lay, other_k]) == 1
    assert "differs" in hb.last_error()
    other_b2, _ = hb.plan(256, 256, 128, 64, "bf16", "idx2", np.zeros((2, 4), np.uint8))
    assert _grouped(L, 2, [lay, other_b2]) == 1
    assert _grouped(L, 2, [lay, lay], ys=[FAKE, None]) == 1         # null output of matrix 1
    assert _grouped(L, 2, [lay, lay], ldys=[256, 100]) == 1         # ldy < n
    assert _grouped(L, 2, [lay, lay], m=0) == 0                    # m == 0: no-op


def test_lowrank_project_rejects(L):
    def call(v=FAKE, ldv=4096, rank=64, k=4096, dtype=hb.HYB_BF16, x=FAKE, m=1, ldx=4096, t=FAKE, ldt=64):
        return L.hyb_lowrank_project(v, ldv, rank, k, dtype, x, m, ldx, t, ldt, None)
    assert call(dtype=hb.HYB_F32) == 3
    assert call(rank=-1) == 2
    assert call(rank=hb.MAX_RANK + 1) == 2
    assert call(k=-8) == 2
    assert call(k=4100) == 2                        # k % 8
    assert call(m=-1) == 2
    assert call(m=16 * 65535 + 1) == 2
    assert call(t=None) == 1
    assert call(ldt=63) == 1
    assert call(v=None) == 1
    assert call(v=FAKE + 8) == 1                    # v alignment
    assert call(ldv=4088) == 1                      # ldv < k
    assert call(ldv=4100) == 1                      # ldv % 8
    assert call(x=None) == 1
    assert call(x=FAKE + 2) == 1
    assert call(ldx=4092) == 1
    assert call(rank=0) == 0                        # no-op
    assert call(m=0) == 0                           # no-op
    assert call(rank=0, t=None, v=None, x=None) == 0


def test_gemv_lowrank_rejects(L):
    lay = _good_layout()
    P = hb.HybPacked(FAKE, FAKE, FAKE, FAKE)

    def call(m=1, t=FAKE, ldt=64, u=FAKE, ldu=64, rank=64, lay=lay):
        return L.hyb_gemv_lowrank(ctypes.byref(lay), ctypes.byref(P), FAKE, m, 256, t, ldt, u, ldu, rank,
                                  FAKE, 3, 256, None)
    assert call(rank=-8) == 2
    assert call(rank=7) == 2                        # rank % 8
    assert call(rank=hb.MAX_RANK + 8) == 2
    assert call(m=17) == 2                          # decode kernel m <= 16
    assert call(t=None) == 1
    assert call(t=FAKE + 4) == 1                    # t alignment
    assert call(ldt=32) == 1                        # ldt < rank
    assert call(ldt=66) == 1                        # ldt % 4
    assert call(u=None) == 1
    assert call(u=FAKE + 8) == 1                    # u alignment
    assert call(ldu=60) == 1                        # ldu < rank
    assert call(ldu=68) == 1                        # ldu % 8
    assert call(m=0, rank=0) == 0                   # rank 0 and m 0: no-op
    assert call(m=0) == 0                           # m 0: no-op
    bad = hb.HybLayout.from_buffer_copy(lay)
    bad.magic = 0
    assert call(lay=bad) == 5
    assert hb.last_error()


def test_gemm_lowrank_rejects(L):
    lay = _good_layout()
    P = hb.HybPacked(FAKE, FAKE, FAKE, FAKE)

    def call(m=40, t=FAKE, ldt=64, u=FAKE, ldu=64, rank=64, ydt=3):
        return L.hyb_gemm_lowrank(ctypes.byref(lay), ctypes.byref(P), FAKE, m, 256, t, ldt, u, ldu, rank,
                                  FAKE, ydt, 256, None)
    assert call(ydt=4) == 3                         # output type
    assert call(rank=12) == 2
    assert call(rank=hb.MAX_RANK + 8) == 2
    assert call(t=None) == 1
    assert call(ldt=66) == 1
    assert call(u=FAKE + 2) == 1
    assert call(ldu=60) == 1
    assert call(m=-1) == 2
    assert call(m=4, t=None) == 1                   # 4 tokens or fewer: the decode entry point's checks
    assert call(m=0) == 0
    assert call(m=4, ydt=2, t=None) == 1
    assert "t is NULL" in hb.last_error()


def test_product_m_zero_is_noop(L):
    lay = _good_layout()
    assert _call(L, "hyb_gemv", lay, m=0, x=None, y=None) == 0
    assert _call(L, "hyb_gemm", lay, m=0, x=None, y=None) == 0


def test_device_tile_sizes(L):
    lay, _ = hb.plan(64, 128, 32, 64, "bf16", "idx2", np.zeros((2, 2), np.uint8))
    assert _call(L, "hyb_gemv", lay, ldx=128, ldy=64) == 4   # b1 = 32 planned but unsupported on device
    P = hb.HybPacked(FAKE, FAKE, FAKE, FAKE)
    assert L.hyb_pack(ctypes.byref(lay), FAKE, 128, ctypes.byref(P), None) == 4
    assert L.hyb_unpack(ctypes.byref(lay), ctypes.byref(P), FAKE, 128, None) == 4


def test_pack_unpack_rejects(L):
    lay = _good_layout()
    P = hb.HybPacked(FAKE, FAKE, FAKE, FAKE)
    assert L.hyb_pack(None, FAKE, 256, ctypes.byref(P), None) == 1
    assert L.hyb_pack(ctypes.byref(lay), None, 256, ctypes.byref(P), None) == 1
    assert L.hyb_pack(ctypes.byref(lay), FAKE, 200, ctypes.byref(P), None) == 1
    assert L.hyb_pack(ctypes.byref(lay), FAKE + 4, 256, ctypes.byref(P), None) == 1
    assert L.hyb_pack(ctypes.byref(lay), FAKE, 256, None, None) == 1
    assert L.hyb_unpack(ctypes.byref(lay), ctypes.byref(P), None, 256, None) == 1
    assert L.hyb_unpack(ctypes.byref(lay), None, FAKE, 256, None) == 1
    bad = hb.HybLayout.from_buffer_copy(lay)
    bad.magic = 1
    assert L.hyb_unpack(ctypes.byref(bad), ctypes.byref(P), FAKE, 256, None) == 5


def test_stream_read_rejects(L):
    assert L.hyb_stream_read(FAKE, -1, FAKE, 1, None) == 2
    assert L.hyb_stream_read(FAKE, 1 << 31, FAKE, 1, None) == 2
    assert L.hyb_stream_read(FAKE, 1024, FAKE, 0, None) == 1
    assert L.hyb_stream_read(FAKE, 1024, FAKE, 65536, None) == 1
    assert L.hyb_stream_read(FAKE, 1024, None, 1, None) == 1
    assert L.hyb_stream_read(None, 1024, FAKE, 1, None) == 1
    assert L.hyb_stream_read(FAKE + 4, 1024, FAKE, 1, None) == 1


def test_product_path_has_no_cpu_fallback():
    """The binding imports nothing from the oracle and raises when the
    library is absent."""
    src = open(os.path.join(ROOT, "matmul_pack_b1_amd", "binding.py")).read()
    assert "oracle" not in src.replace("no CPU fallback", "")
    for name in os.listdir(os.path.join(ROOT, "matmul_pack_b1_amd")):
        if name.endswith(".py"):
            text = open(os.path.join(ROOT, "matmul_pack_b1_amd", name)).read()
            assert "import oracle" not in text and "from oracle" not in text, name


# -------------------------------------------------- kernel routing --------

def _layout(n, k, b):
    L, _ = hb.plan(n, k, b, b, "bf16", "idx2", np.zeros((n // b, k // b), np.uint8))
    return L


# (n, k, tile, m) -> (kernel, token blocks, wavefronts, row groups) on a
# 256-CU device (the MI355X; also the count assumed when no device is
# visible).  These are the routes the GPU parity tests' docstrings name.
ROUTES = [
    ((14336, 4096, 128, 1), ("decode", 0, 4, 0)),
    ((1024, 4096, 128, 16), ("decode", 0, 16, 0)),       # short matrix: decode kernel up to 16 tokens
    ((4096, 14336, 128, 8), ("decode", 0, 16, 0)),       # one 16-row slab per CU
    ((14336, 4096, 128, 4), ("decode", 0, 4, 0)),
    ((14336, 4096, 128, 5), ("register", 1, 8, 1)),      # 5-16 tokens on the matrix cores
    ((5120, 17408, 64, 12), ("split", 1, 8, 1)),         # 320 slabs: matrix cores from 5 tokens
    ((14336, 4096, 128, 12), ("register", 1, 8, 1)),
    ((17408, 5120, 64, 12), ("split", 1, 4, 1)),         # 272 64-row groups: K split over 256 workgroups
    ((17408, 5120, 64, 16), ("split", 1, 4, 1)),
    ((17408, 5120, 64, 40), ("split", 3, 4, 2)),         # 136 tiles of 128 rows x 48 tokens on 256 CUs
    ((17408, 5120, 64, 64), ("split", 4, 8, 4)),         # the LDS-fed 64-token shape, split
    ((17408, 5120, 64, 96), ("split", 3, 4, 2)),
    ((17408, 5120, 64, 100), ("split", 8, 8, 4)),        # 68 LDS 128-token tiles split over 256 workgroups
    ((17408, 5120, 64, 128), ("split", 8, 8, 4)),
    ((8256, 5120, 64, 100), ("split", 4, 8, 4)),         # last 256-row block a quarter full
    ((28672, 8192, 128, 64), ("register", 4, 4, 2)),     # one round of 224 tiles: no split
    ((4096, 14336, 128, 256), ("split", 16, 8, 4)),      # 16 LDS 256-token tiles, K cut in 14 parts
    ((4096, 14336, 128, 160), ("split", 3, 4, 2)),       # register-fed split
    ((14336, 4096, 128, 64), ("register", 2, 4, 2)),
    ((14336, 4096, 128, 128), ("register", 4, 4, 2)),    # 224 tiles fill the CUs well enough
    ((28672, 8192, 128, 96), ("split", 3, 4, 2)),        # split 48-token tiles beat one LDS round
    ((28672, 8192, 128, 128), ("split", 8, 8, 4)),
    ((28672, 8192, 128, 256), ("lds", 8, 8, 4)),         # 224 tiles of 128 tokens: one round
    ((8192, 28672, 128, 16), ("split", 1, 8, 1)),        # 128 groups on 256 CUs, 448 K steps
    ((8192, 28672, 128, 64), ("split", 4, 4, 2)),
    ((8192, 28672, 128, 128), ("split", 8, 8, 4)),
    ((1024, 4096, 128, 32), ("split", 1, 8, 1)),
    ((17408, 5120, 64, 2048), ("split", 16, 8, 4)),      # 2 rounds of 256-token tiles, then 32 tiles in 5 K parts
    ((17408, 5120, 64, 1024), ("split", 16, 8, 4)),      # 1 round, then 16 tiles in 5 K parts
    ((17408, 5120, 64, 1536), ("lds", 16, 8, 4)),        # a tail of 156 tiles has no room for 2 parts
    ((17408, 5120, 64, 3072), ("split", 16, 8, 4)),
    ((28672, 8192, 128, 2048), ("split", 16, 8, 4)),
    ((28672, 8192, 128, 1536), ("lds", 16, 8, 4)),
    ((14336, 4096, 128, 4096), ("split", 16, 8, 4)),
    ((16640, 4096, 128, 1024), ("split", 16, 8, 4)),     # 1 round, then 4 tiles in 4 K parts
    ((14336, 4096, 128, 200), ("split", 16, 8, 4)),
    ((14336, 4096, 128, 160), ("split", 12, 8, 4)),      # 192-token tiles, K cut in 4 parts
    ((14336, 4096, 128, 300), ("lds", 8, 8, 4)),
    ((14336, 4096, 128, 700), ("lds", 12, 8, 4)),
    ((14336, 4096, 128, 1024), ("lds", 16, 8, 4)),
    ((14336, 4096, 128, 2048), ("lds", 16, 8, 4)),
    ((8192, 28672, 128, 256), ("split", 16, 8, 4)),      # few 256-row blocks
    ((8192, 28672, 128, 384), ("split", 12, 8, 4)),
    ((8192, 28672, 128, 512), ("split", 16, 8, 4)),
    ((8192, 28672, 128, 1024), ("split", 16, 8, 4)),     # 128 256-token tiles, K cut in halves
    ((8192, 28672, 128, 2048), ("lds", 16, 8, 4)),       # 256 tiles of 256 tokens: one full round
    ((4096, 4096, 128, 160), ("register", 2, 4, 2)),
    ((1024, 4096, 128, 384), ("register", 2, 8, 1)),
    ((8192, 256, 64, 1024), ("lds", 8, 8, 4)),
    ((8192, 256, 64, 2048), ("lds", 16, 8, 4)),
    ((16384, 256, 64, 256), ("lds", 4, 8, 4)),
    ((64, 64, 64, 4_300_000), ("lds", 16, 8, 4)),        # register-fed grids would exceed 65535 blocks
]


@pytest.mark.parametrize("case,expect", ROUTES)
def test_gemm_routes(case, expect):
    n, k, b, m = case
    got = hb.gemm_shape(_layout(n, k, b), m)
    assert (got["kernel"], got["token_blocks"], got["waves"], got["row_groups"]) == expect, got


def test_split_workspace_sizes(L):
    """hyb_gemm_workspace_size: 2 pieces (1 for the K-parts routes) x (rows x
    tokens x 4 bytes) per workgroup of a split route, 0 for every other route and for m = 0;
    never above the 64 MiB the library holds per stream."""
    for (n, k, b, m), expect in ROUTES:
        lay = _layout(n, k, b)
        size = ctypes.c_size_t(7)
        assert L.hyb_gemm_workspace_size(ctypes.byref(lay), m, ctypes.byref(size)) == 0
        if expect[0] == "split":
            _, mb, _, rg = expect
            # two partial tiles per stream-K workgroup, one per workgroup of
            # the 192- and 256-token LDS tiles (K cut into equal parts)
            pieces = 1 if (rg == 4 and mb >= 12) else 2
            tiles_per_group = pieces * (64 * rg) * (16 * mb) * 4
            assert size.value > 0 and size.value % tiles_per_group == 0, (n, k, m, size.value)
            assert size.value // tiles_per_group <= 256
            assert size.value <= 64 << 20
        else:
            assert size.value == 0, (n, k, m)
    lay = _layout(17408, 5120, 64)
    size = ctypes.c_size_t(7)
    assert L.hyb_gemm_workspace_size(ctypes.byref(lay), 0, ctypes.byref(size)) == 0 and size.value == 0
    # whole rounds of 256-token tiles, then the last row blocks in K parts:
    # only the parts hold partial tiles (256 rows x 256 tokens x 4 bytes each)
    for (n, k, b, m), tail_wgs in [((17408, 5120, 64, 2048), 32 * 5), ((17408, 5120, 64, 1024), 16 * 5),
                                   ((17408, 5120, 64, 4096), 64 * 4), ((28672, 8192, 128, 2048), 128 * 2),
                                   ((16640, 4096, 128, 1024), 4 * 4)]:
        assert L.hyb_gemm_workspace_size(ctypes.byref(_layout(n, k, b)), m, ctypes.byref(size)) == 0
        assert size.value == tail_wgs * 256 * 256 * 4, (n, k, m, size.value)
    assert L.hyb_gemm_workspace_size(ctypes.byref(lay), -1, ctypes.byref(size)) == 2
    assert L.hyb_gemm_workspace_size(ctypes.byref(lay), 100, None) == 1
    assert L.hyb_gemm_workspace_size(None, 100, ctypes.byref(size)) == 1


def test_gemm_ws_rejects_before_launch(L):
    """hyb_gemm_ws: a positive size with a NULL or misaligned workspace, or a
    size below the need, is HYB_ERR_INVALID_ARG before anything runs."""
    fn = L.hyb_gemm_ws
    L2, _ = hb.plan(2048, 16384, 128, 128, "bf16", "idx2", np.zeros((16, 128), np.uint8))
    need = ctypes.c_size_t(0)
    assert L.hyb_gemm_workspace_size(ctypes.byref(L2), 100, ctypes.byref(need)) == 0 and need.value > 0
    packed = hb.HybPacked(FAKE, FAKE, FAKE, FAKE)
    args = lambda ws, nb: (ctypes.byref(L2), ctypes.byref(packed), FAKE, 100, 16384, FAKE, 3, 2048, ws, nb, None)
    assert fn(*args(None, need.value)) == 1                 # NULL with a size
    assert fn(*args(FAKE + 8, need.value)) == 1             # misaligned
    assert fn(*args(FAKE, need.value - 16)) == 1            # below the need


def test_gemm_lowrank_ws_rejects_before_launch(L):
    """hyb_gemm_lowrank_ws: the workspace checks of hyb_gemm_ws (NULL or
    misaligned with a size, a size below the need) and a NULL t are
    HYB_ERR_INVALID_ARG, a rank off the multiple-of-8 grid HYB_ERR_SHAPE,
    all before anything runs."""
    fn = L.hyb_gemm_lowrank_ws
    L2, _ = hb.plan(2048, 16384, 128, 128, "bf16", "idx2", np.zeros((16, 128), np.uint8))
    need = ctypes.c_size_t(0)
    assert L.hyb_gemm_workspace_size(ctypes.byref(L2), 100, ctypes.byref(need)) == 0 and need.value > 0
    packed = hb.HybPacked(FAKE, FAKE, FAKE, FAKE)
    args = lambda ws, nb, t=FAKE, rank=16: (ctypes.byref(L2), ctypes.byref(packed), FAKE, 100, 16384, t, 16, FAKE, 16,
                                            rank, FAKE, 3, 2048, ws, nb, None)
    assert fn(*args(None, need.value)) == 1                 # NULL with a size
    assert fn(*args(FAKE + 8, need.value)) == 1             # misaligned
    assert fn(*args(FAKE, need.value - 16)) == 1            # below the need
    assert fn(*args(FAKE, need.value, t=None)) == 1         # t NULL
    assert fn(*args(FAKE, need.value, rank=12)) == 2        # rank not a multiple of 8: HYB_ERR_SHAPE


def test_gemm_shape_rejects(L):
    lay = _layout(1024, 1024, 128)
    out = (ctypes.c_int32 * 4)()
    assert L.hyb_gemm_shape(ctypes.byref(lay), 0, ctypes.byref(out)) == 2   # m < 1
    assert L.hyb_gemm_shape(ctypes.byref(lay), 8, None) == 1                # out NULL
    assert L.hyb_gemm_shape(None, 8, ctypes.byref(out)) == 1                # layout NULL
    bad = hb.HybLayout.from_buffer_copy(lay)
    bad.magic = 0
    assert L.hyb_gemm_shape(ctypes.byref(bad), 8, ctypes.byref(out)) == 5   # HYB_ERR_FORMAT


# ------------------------------------------- strides and the m limit -------

def test_negative_strides_rejected_even_when_empty(L):
    """A negative row stride is an invalid argument even when the operand is
    empty (k = 0 or n = 0): the kernels size buffer ranges as rows * stride."""
    lay_k0, _ = hb.plan(256, 0, 128, 128, "bf16", "idx2", np.zeros((2, 0), np.uint8))
    for fn in ("hyb_gemv", "hyb_gemm", "hyb_gemm_mfma", "hyb_gemm_noalloc"):
        assert _call(L, fn, lay_k0, m=20 if fn != "hyb_gemv" else 4, ldx=-8) == 1, fn
    lay_n0, _ = hb.plan(0, 256, 128, 128, "bf16", "idx2", np.zeros((0, 2), np.uint8))
    packed = hb.HybPacked(None, None, None, None)
    assert L.hyb_pack(ctypes.byref(lay_n0), FAKE, -8, ctypes.byref(packed), None) == 1
    assert L.hyb_unpack(ctypes.byref(lay_n0), ctypes.byref(packed), FAKE, -8, None) == 1
    good = _good_layout()
    assert _call(L, "hyb_gemm", good, m=40, ldx=-256) == 1


def test_gemm_shape_applies_the_launch_limit():
    """hyb_gemm_shape reports HYB_ERR_UNSUPPORTED where hyb_gemm_mfma would
    reject the token count, instead of a register-fed shape computed from an
    overflowed block count."""
    lay = _layout(64, 64, 64)
    for m in (2**31 - 1, 2**31 - 40, 16 * 65535 * 8 + 1):
        with pytest.raises(hb.HybError) as e:
            hb.gemm_shape(lay, m)
        assert e.value.status == 4, m
    got = hb.gemm_shape(lay, 16 * 65535 * 8)
    assert got["kernel"] == "lds"


# ------------------------------------- binding checks before any launch ----

class _NoLaunch:
    """Stands in for the library: host planning passes through, any device
    entry point fails the test."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in ("hyb_plan", "hyb_status_str", "hyb_last_error"):
            return getattr(self._real, name)
        raise AssertionError(f"{name} reached although the arguments are invalid")


@pytest.fixture()
def cpu_weight(monkeypatch):
    torch = pytest.importorskip("torch")
    real = hb.lib()
    n, k, b = 256, 256, 128
    tmap = np.array([[1, 0], [0, 1]], np.uint8)
    lay, tidx = hb.plan(n, k, b, b, "bf16", "idx2", tmap)
    P = hb.allocate(lay, tidx, torch.device("cpu"), "bf16", "idx2")
    monkeypatch.setattr(hb, "_lib", _NoLaunch(real))
    return torch, P, tmap


def test_binding_rejects_bad_x(cpu_weight):
    torch, P, _ = cpu_weight
    with pytest.raises(ValueError, match="columns"):
        hb.gemv(P, torch.zeros((1, 255), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="weight is bf16"):
        hb.gemm(P, torch.zeros((3, 256), dtype=torch.float16))
    with pytest.raises(TypeError, match="weight is bf16"):
        hb.gemv(P, torch.zeros((1, 256), dtype=torch.float32))


def test_binding_rejects_bad_out(cpu_weight):
    torch, P, _ = cpu_weight
    x = torch.zeros((2, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"expected \(2, 256\)"):
        hb.gemv(P, x, out=torch.empty((1, 256), dtype=torch.float32))
    with pytest.raises(ValueError, match=r"expected \(2, 256\)"):
        hb.gemm_mfma(P, x, out=torch.empty((2, 300), dtype=torch.float32))
    with pytest.raises(TypeError, match="expected torch.float32"):
        hb.gemm(P, x, out_dtype=torch.float32, out=torch.empty((2, 256), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="must be float32 or the weight dtype"):
        hb.gemv(P, x, out=torch.empty((2, 256), dtype=torch.float16))
    with pytest.raises(ValueError, match=r"expected \(256, 256\)"):
        hb.unpack(P, out=torch.empty((256, 128), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="expected torch.bfloat16"):
        hb.unpack(P, out=torch.empty((256, 256), dtype=torch.float16))


def test_binding_rejects_bad_pack_target(cpu_weight):
    torch, P, tmap = cpu_weight
    with pytest.raises(ValueError, match="out holds 256x256"):
        hb.pack(torch.zeros((128, 256), dtype=torch.bfloat16), tmap[:1], 128, 128, out=P)
    with pytest.raises(TypeError, match="out holds bf16/idx2"):
        hb.pack(torch.zeros((256, 256), dtype=torch.float16), tmap, 128, 128, out=P)
    with pytest.raises(ValueError, match="tile map does not match"):
        hb.pack(torch.zeros((256, 256), dtype=torch.bfloat16), np.ones((2, 2), np.uint8), 128, 128, out=P)


def test_binding_rejects_bad_grouped_and_lowrank(cpu_weight):
    torch, P, _ = cpu_weight
    x = torch.zeros((1, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="columns"):
        hb.gemv_grouped([P, P], torch.zeros((1, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match=r"outs\[1\]"):
        hb.gemv_grouped([P, P], x, outs=[torch.empty((1, 256)), torch.empty((2, 256))])
    t = torch.zeros((1, 8), dtype=torch.float32)
    with pytest.raises(TypeError, match="u is torch.float16"):
        hb.gemv_lowrank(P, x, t, torch.zeros((256, 8), dtype=torch.float16))
    with pytest.raises(ValueError, match="u 256 x rank"):
        hb.gemm_lowrank(P, x, t, torch.zeros((256, 16), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match=r"expected \(1, 8\)"):
        hb.lowrank_project(torch.zeros((8, 256), dtype=torch.bfloat16), x, out=torch.empty((1, 16)))


# ------------------------------------------------------- save / load -------

def test_layout_check(L):
    lay = _good_layout()
    assert L.hyb_layout_check(ctypes.byref(lay)) == 0
    assert L.hyb_layout_check(None) == 1
    for field, value in (("magic", 0x31425949), ("version", 2), ("val_bytes", lay.val_bytes + 16),
                         ("n_sparse", lay.n_sparse + 1), ("tidx_bytes", 0)):
        bad = hb.HybLayout.from_buffer_copy(lay)
        setattr(bad, field, value)
        assert L.hyb_layout_check(ctypes.byref(bad)) == 5, field
    bad = hb.HybLayout.from_buffer_copy(lay)
    bad.dtype = 9
    assert L.hyb_layout_check(ctypes.byref(bad)) == 3


def test_save_load_round_trip_and_rejections(tmp_path):
    """A packed weight written by save() reads back byte for byte; a header
    with the wrong magic or version is refused with HYB_ERR_FORMAT, and a
    short or overlong file with ValueError, before anything is allocated."""
    torch = pytest.importorskip("torch")
    n, k, b = 256, 384, 128
    rng = np.random.default_rng(12)
    tmap = (rng.random((n // b, k // b)) < 0.5).astype(np.uint8)
    lay, tidx = hb.plan(n, k, b, b, "f16", "mask4", tmap)
    P = hb.allocate(lay, tidx, torch.device("cpu"), "f16", "mask4")
    for t in (P.dense, P.val, P.meta):
        t.copy_(torch.from_numpy(rng.integers(0, 256, t.numel(), dtype=np.uint8)))
    path = tmp_path / "w.hyb"
    hb.save(P, path)
    assert path.stat().st_size == ctypes.sizeof(hb.HybLayout) + lay.dense_bytes + lay.val_bytes + lay.meta_bytes + lay.tidx_bytes
    Q = hb.load(path, torch.device("cpu"))
    assert bytes(Q.layout) == bytes(P.layout)
    assert (Q.dtype, Q.meta_kind) == ("f16", "mask4")
    for name in ("dense", "val", "meta", "tidx"):
        assert torch.equal(getattr(Q, name), getattr(P, name)), name
    raw = path.read_bytes()
    for offset, value in ((0, b"HYB2"), (4, (2).to_bytes(4, "little"))):
        bad = tmp_path / f"bad{offset}.hyb"
        bad.write_bytes(raw[:offset] + value + raw[offset + 4:])
        with pytest.raises(hb.HybError) as e:
            hb.load(bad, torch.device("cpu"))
        assert e.value.status == 5
    short = tmp_path / "short.hyb"
    short.write_bytes(raw[:-4])
    with pytest.raises(ValueError, match="truncated"):
        hb.load(short, torch.device("cpu"))
    long_ = tmp_path / "long.hyb"
    long_.write_bytes(raw + b"\0")
    with pytest.raises(ValueError, match="trailing"):
        hb.load(long_, torch.device("cpu"))
