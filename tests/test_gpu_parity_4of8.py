"""GPU parity of the 4:8 sparse tiles (metadata kind mask8): pack / unpack
bit-exact against the oracle, every product path within the same bound as
the 2:4 tiles (|y - y_ref| <= 2e-3 * s), bitwise closed forms, and the
grouped and low-rank decode entry points.  The matrix-core tests pick token
counts and shapes that reach each kernel variant: the decode kernel (m <= 4
through hyb_gemm), the register-fed kernel with eight and four wavefronts,
two row groups per workgroup (17408 rows: more 64-row groups than compute
units), 65-128 tokens, and the four LDS-fed shapes (17408 rows at 256 and
2048 tokens, and 8192 or 16384 rows at 256-2048)."""
import numpy as np
import pytest

import oracle
from matmul_pack_b1_amd import binding as hb
from matmul_pack_b1_amd import workloads as wl
from tests.test_gpu_parity import (_torch, assert_close, note, oracle_full, pack_gpu, random_case, sample_tile_rows, streams,
                                   upload, workload_matrix)

pytestmark = pytest.mark.gpu

META = "mask8"


def _prune(w, tmap, b1, b2):
    return oracle.prune(w, tmap, b1, b2, META)


@pytest.mark.parametrize("b1,b2", [(64, 64), (64, 128), (128, 128), (128, 256), (256, 64), (256, 256)])
def test_pack_unpack_4of8_random(b1, b2):
    dtype = "bf16" if b2 != 256 else "f16"
    note(f"pack 4:8 random {b1}x{b2} {dtype}")
    w, tmap = random_case(b1 + b2 + 8, 3 * b1, 3 * b2, b1, b2, dtype)
    rng = np.random.default_rng(8)
    for v in (0x8000, 0x0000, 0x0001, 0x8003, 0x7C00 if dtype == "f16" else 0x7F80, 0xFFC0):
        w[rng.random(w.shape) < 0.03] = v
    P = pack_gpu(w, tmap, b1, b2, dtype, META)
    ref = oracle.pack(w, tmap, b1, b2, META)
    got = streams(P)
    for key in ("dense", "val", "meta", "tidx"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    u = hb.tensor_to_bits(hb.unpack(P))
    np.testing.assert_array_equal(u, _prune(w, tmap, b1, b2))


def test_pack_unpack_4of8_workload():
    mat, w, tmap = workload_matrix(2, 0)
    note(f"pack 4:8 workload {mat.name}")
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, META)
    ref = oracle.pack(w, tmap, mat.b1, mat.b2, META)
    got = streams(P)
    for key in ("dense", "val", "meta", "tidx"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    u = hb.tensor_to_bits(hb.unpack(P))
    np.testing.assert_array_equal(u, _prune(w, tmap, mat.b1, mat.b2))


@pytest.mark.parametrize("m", [1, 3, 8, 16])
@pytest.mark.parametrize("b1,b2,dtype", [(64, 64, "bf16"), (128, 256, "f16"), (256, 128, "bf16")])
def test_gemv_4of8_random(m, b1, b2, dtype):
    torch = _torch()
    note(f"gemv 4:8 m={m} {b1}x{b2} {dtype}")
    w, tmap = random_case(m * 5 + b2 + 48, 2 * b1, 5 * b2, b1, b2, dtype)
    x = wl.float32_to_bits(np.random.default_rng(m + 48).standard_normal((m, 5 * b2)).astype(np.float32), dtype)
    P = pack_gpu(w, tmap, b1, b2, dtype, META)
    y = hb.gemv(P, upload(x, dtype))
    torch.cuda.synchronize()
    yref, s = oracle.ref_matmul(_prune(w, tmap, b1, b2), x, dtype)
    assert_close(y.cpu().numpy(), yref, s, what="gemv 4:8")


@pytest.mark.parametrize("m", [1, 16])
def test_gemv_4of8_workload(m):
    mat, w, tmap = workload_matrix(2, 0)
    note(f"gemv 4:8 workload m={m}")
    x = mat.activation_bits(m)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, META)
    y = hb.gemv(P, upload(x, mat.dtype)).cpu().numpy()
    yref, s = oracle.ref_matmul(_prune(w, tmap, mat.b1, mat.b2), x, mat.dtype)
    assert_close(y, yref, s, what=f"gemv 4:8 m={m}")


@pytest.mark.parametrize("m", [9, 17, 40, 64, 100, 130, 257, 600])
@pytest.mark.parametrize("b1,b2,dtype", [(64, 64, "bf16"), (128, 128, "f16"), (64, 256, "bf16")])
def test_gemm_4of8_random(m, b1, b2, dtype):
    torch = _torch()
    note(f"gemm 4:8 m={m} {b1}x{b2} {dtype}")
    n, k = 4 * b1, 3 * b2
    w, tmap = random_case(m + b1 + b2 + 48, n, k, b1, b2, dtype)
    x = wl.float32_to_bits(np.random.default_rng(m).standard_normal((m, k)).astype(np.float32), dtype)
    P = pack_gpu(w, tmap, b1, b2, dtype, META)
    y = hb.gemm(P, upload(x, dtype))
    torch.cuda.synchronize()
    yref, s = oracle.ref_matmul(_prune(w, tmap, b1, b2), x, dtype)
    assert_close(y.cpu().numpy(), yref, s, what="gemm 4:8")


@pytest.mark.parametrize("n,m", [(8192, 1024), (8192, 2048), (16384, 256)])
@pytest.mark.parametrize("b1,b2,dtype", [(64, 64, "bf16"), (128, 128, "f16"), (64, 256, "bf16")])
def test_gemm_4of8_lds_shapes_random(n, m, b1, b2, dtype):
    """The LDS-fed shapes (128-, 256- and 64-token workgroups on a 256-CU
    device) on 4:8 tiles in each tile size and dtype; the small matrices of
    test_gemm_4of8_random take the register-fed kernel at every token
    count.  Every output against the oracle."""
    torch = _torch()
    note(f"gemm 4:8 lds shapes n={n} m={m} {b1}x{b2} {dtype}")
    k = 2 * b2
    w, tmap = random_case(n + m + b2 + 8, n, k, b1, b2, dtype)
    x = wl.float32_to_bits(np.random.default_rng(m + n + 8).standard_normal((m, k)).astype(np.float32), dtype)
    P = pack_gpu(w, tmap, b1, b2, dtype, META)
    y = hb.gemm(P, upload(x, dtype)).cpu().numpy()
    yref, s = oracle_full(w, tmap, b1, b2, x, dtype, meta=META)
    assert_close(y, yref, s, what=f"4:8 lds shapes n={n} m={m}")


@pytest.mark.parametrize("m", [4, 12, 30, 64, 100, 256, 2048])
def test_gemm_4of8_qwen14b(m):
    """17408 x 5120, 64 x 64 tiles, 60% of them 4:8: full-size launches
    (272 row groups of 64, more than the compute units), every output
    against the oracle."""
    mat, w, tmap = workload_matrix(5, 0)
    note(f"gemm 4:8 qwen14b m={m}")
    x = mat.activation_bits(m)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, META)
    y = hb.gemm(P, upload(x, mat.dtype)).cpu().numpy()
    yref, s = oracle_full(w, tmap, mat.b1, mat.b2, x, mat.dtype, meta=META)
    assert_close(y, yref, s, what=f"qwen14b 4:8 m={m}")


@pytest.mark.parametrize("kernel", ["gemv", "gemm_mfma"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_one_hot_columns_exact_4of8(kernel, dtype):
    """x = e_c gives column c of W' bit for bit, with the 4:8 expansion."""
    torch = _torch()
    note(f"one-hot 4:8 {kernel} {dtype}")
    b1, b2 = 64, 128
    w, tmap = random_case(21, 2 * b1, 2 * b2, b1, b2, dtype)
    w[::7, ::5] = 0x0001
    cols = np.array([0, 1, 7, 8, 63, 64, 100, 127, 128, 255])
    one = 0x3F80 if dtype == "bf16" else 0x3C00
    m = len(cols) if kernel == "gemv" else 32
    x = np.zeros((m, 2 * b2), np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = one
    P = pack_gpu(w, tmap, b1, b2, dtype, META)
    fn = hb.gemv if kernel == "gemv" else hb.gemm_mfma
    y = fn(P, upload(x, dtype)).cpu().numpy()
    wp = _prune(w, tmap, b1, b2)
    for i, c in enumerate(cols):
        np.testing.assert_array_equal(y[i], oracle.widen(wp[:, c], dtype).astype(np.float32))
    assert np.all(y[len(cols):] == 0)


@pytest.mark.parametrize("kernel", ["gemv", "gemm_mfma"])
def test_small_integers_exact_4of8(kernel):
    note(f"integers 4:8 {kernel}")
    rng = np.random.default_rng(22)
    b1, b2 = 128, 64
    n, k, m = 256, 640, (5 if kernel == "gemv" else 150)
    w = wl.float32_to_bits(rng.integers(-3, 4, size=(n, k)).astype(np.float32), "bf16")
    x = wl.float32_to_bits(rng.integers(-3, 4, size=(m, k)).astype(np.float32), "bf16")
    tmap = (rng.random((n // b1, k // b2)) < 0.5).astype(np.uint8)
    P = pack_gpu(w, tmap, b1, b2, "bf16", META)
    fn = hb.gemv if kernel == "gemv" else hb.gemm_mfma
    y = fn(P, upload(x, "bf16")).cpu().numpy()
    yref, _ = oracle.ref_matmul(_prune(w, tmap, b1, b2), x, "bf16")
    np.testing.assert_array_equal(y.astype(np.float64), yref)


def test_4of8_differs_from_2of4():
    """The same weight packed 4:8 and 2:4 gives different W' (and products
    that each match their own oracle), so the 4:8 path is not a relabelled
    2:4 path."""
    torch = _torch()
    note("4:8 vs 2:4")
    w, tmap = random_case(23, 128, 256, 64, 128, "bf16")
    x = wl.float32_to_bits(np.random.default_rng(23).standard_normal((3, 256)).astype(np.float32), "bf16")
    y8 = hb.gemv(pack_gpu(w, tmap, 64, 128, "bf16", META), upload(x, "bf16")).cpu().numpy()
    y4 = hb.gemv(pack_gpu(w, tmap, 64, 128, "bf16", "idx2"), upload(x, "bf16")).cpu().numpy()
    torch.cuda.synchronize()
    w8, w4 = _prune(w, tmap, 64, 128), oracle.prune(w, tmap, 64, 128)
    assert np.any(w8 != w4)
    r8, s8 = oracle.ref_matmul(w8, x, "bf16")
    r4, s4 = oracle.ref_matmul(w4, x, "bf16")
    assert_close(y8, r8, s8, what="4:8")
    assert_close(y4, r4, s4, what="2:4")
    assert np.any(y8 != y4)


def test_gemv_grouped_and_lowrank_4of8():
    """The grouped launch over two 4:8 matrices equals separate launches
    bitwise; the low-rank epilogue on a 4:8 weight matches the oracle."""
    torch = _torch()
    note("grouped + low-rank 4:8")
    wa, ta = random_case(24, 256, 512, 128, 128, "bf16")
    wb, tb = random_case(25, 128, 512, 64, 128, "bf16", frac=0.8)
    x = wl.float32_to_bits(np.random.default_rng(24).standard_normal((4, 512)).astype(np.float32), "bf16")
    Pa = pack_gpu(wa, ta, 128, 128, "bf16", META)
    Pb = pack_gpu(wb, tb, 64, 128, "bf16", META)
    xt = upload(x, "bf16")
    ya, yb = hb.gemv_grouped([Pa, Pb], xt)
    assert torch.equal(ya, hb.gemv(Pa, xt)) and torch.equal(yb, hb.gemv(Pb, xt))
    rng = np.random.default_rng(26)
    t = rng.standard_normal((4, 64)).astype(np.float32)
    u = wl.float32_to_bits(rng.standard_normal((256, 64)).astype(np.float32) * 0.05, "bf16")
    y = hb.gemv_lowrank(Pa, xt, torch.from_numpy(t).to(xt.device), upload(u, "bf16")).cpu().numpy()
    yref, s = oracle.ref_lowrank(_prune(wa, ta, 128, 128), x, t, u, "bf16")
    assert_close(y, yref, s, what="low-rank 4:8")


def test_corrupt_tile_index_is_skipped_4of8():
    torch = _torch()
    note("corrupt tidx 4:8")
    w, tmap = random_case(27, 128, 256, 64, 128, "bf16")
    P = pack_gpu(w, tmap, 64, 128, "bf16", META)
    bad = P.tidx.cpu().numpy().copy()
    bad[0] = 1 << 30
    bad[-1] = -(1 << 30)
    P.tidx.copy_(torch.from_numpy(bad))
    x = wl.float32_to_bits(np.random.default_rng(4).standard_normal((2, 256)).astype(np.float32), "bf16")
    y = hb.gemv(P, upload(x, "bf16")).cpu().numpy()
    y2 = hb.gemm_mfma(P, upload(x, "bf16")).cpu().numpy()
    wp = _prune(w, tmap, 64, 128)
    wp[0:64, 0:128] = 0
    wp[64:128, 128:256] = 0
    yref, s = oracle.ref_matmul(wp, x, "bf16")
    assert_close(y, yref, s, what="gemv corrupt 4:8")
    assert_close(y2, yref, s, what="gemm corrupt 4:8")
