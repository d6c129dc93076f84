"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on
the same seeded inputs.

Bars: pack / unpack bit-exact; products within |y - y_ref| <= 2e-3 * s per
element (s = sum_k |w x|), plus bitwise closed forms (one-hot, small
integers, zero input).  Every output of every workload matrix is checked;
the oracle prunes and multiplies large matrices a chunk of tile rows at a
time.  Tests that name a kernel route assert it with hyb_gemm_shape."""
import functools
import sys

import numpy as np
import pytest

import oracle
from matmul_pack_b1_amd import binding as hb
from matmul_pack_b1_amd import workloads as wl

pytestmark = pytest.mark.gpu

REL = 2e-3


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    return _torch().device("cuda:0")


def upload(bits, dtype):
    return hb.bits_to_tensor(bits, dtype, dev())


def assert_close(y, yref, s, extra=0.0, what=""):
    """The acceptance rule of the oracle (|y - y_ref| <= 2e-3 * s + extra)."""
    y = np.asarray(y, dtype=np.float64)
    bad = ~oracle.within_bound(y, yref, s, REL, extra)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside bound; first at {tuple(i)}: "
                             f"y={y[tuple(i)]!r} ref={yref[tuple(i)]!r} s={s[tuple(i)]!r}")


def pack_gpu(w_bits, tmap, b1, b2, dtype, meta):
    torch = _torch()
    w = upload(w_bits, dtype)
    P = hb.pack(w, tmap, b1, b2, meta)
    torch.cuda.synchronize()
    return P


def streams(P):
    return {
        "dense": P.dense.cpu().numpy().view(np.uint16),
        "val": P.val.cpu().numpy().view(np.uint16),
        "meta": P.meta.cpu().numpy(),
        "tidx": P.tidx.cpu().numpy(),
    }


def random_case(seed, n, k, b1, b2, dtype, frac=0.5, sigma=0.02):
    rng = np.random.default_rng(seed)
    w = wl.float32_to_bits(rng.standard_normal((n, k)).astype(np.float32) * sigma, dtype)
    tmap = (rng.random((n // b1, k // b2)) < frac).astype(np.uint8)
    return w, tmap


@functools.lru_cache(maxsize=4)
def workload_matrix(config, index):
    mat = wl.workload(config).matrices[index]
    return mat, mat.weight_bits(), mat.tile_map()


def sample_tile_rows(mat, count, seed=0):
    rng = np.random.default_rng(seed)
    tn = mat.n // mat.b1
    return np.sort(rng.choice(tn, size=min(count, tn), replace=False))


def oracle_full(w_bits, tmap, b1, b2, x_bits, dtype, meta="idx2", chunk_rows=2048):
    """Oracle y/s for every output row.  Tile rows are pruned and multiplied
    a chunk at a time (pruning acts tile by tile, so the chunks give exactly
    the rows of the whole), which bounds host memory at the 70B shapes."""
    n = w_bits.shape[0]
    step = max(b1, (chunk_rows // b1) * b1)
    ys, ss = [], []
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        sub = oracle.prune(w_bits[r0:r1], tmap[r0 // b1:r1 // b1], b1, b2, meta)
        y, s = oracle.ref_matmul(sub, x_bits, dtype)
        ys.append(y)
        ss.append(s)
    return np.concatenate(ys, axis=1), np.concatenate(ss, axis=1)


def oracle_full_lowrank(w_bits, tmap, b1, b2, x_bits, t, u_bits, dtype, meta="idx2", chunk_rows=2048):
    """oracle.ref_lowrank for every output row, a chunk of tile rows at a
    time (as oracle_full)."""
    n = w_bits.shape[0]
    step = max(b1, (chunk_rows // b1) * b1)
    ys, ss = [], []
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        sub = oracle.prune(w_bits[r0:r1], tmap[r0 // b1:r1 // b1], b1, b2, meta)
        y, s = oracle.ref_lowrank(sub, x_bits, t, u_bits[r0:r1], dtype)
        ys.append(y)
        ss.append(s)
    return np.concatenate(ys, axis=1), np.concatenate(ss, axis=1)


def device_cus():
    return _torch().cuda.get_device_properties(0).multi_processor_count


def expect_route(P, m, kernel, token_blocks=None, waves=None, row_groups=None):
    """Assert the kernel and shape hyb_gemm launches for m tokens (the route
    a test's docstring names).  The route table was measured on a 256-CU
    device; on another CU count a different route is legitimate, and the
    test is skipped rather than run on a kernel it does not claim to cover."""
    got = hb.gemm_shape(P.layout, m)
    want = {"kernel": kernel, "token_blocks": token_blocks, "waves": waves, "row_groups": row_groups}
    want = {k: v for k, v in want.items() if v is not None}
    same = all(got[k] == v for k, v in want.items())
    if device_cus() != 256 and not same:
        pytest.skip(f"route measured on 256 CUs; this device has {device_cus()} and runs {got}")
    assert same, f"m={m}: expected {want}, hyb_gemm_shape gives {got}"


def oracle_rows(w_bits, tmap, mat, tile_rows, x_bits):
    """Oracle y/s for the rows of the chosen tile rows only."""
    rows = np.concatenate([np.arange(t * mat.b1, (t + 1) * mat.b1) for t in tile_rows])
    sub = oracle.prune(w_bits[rows], tmap[tile_rows], mat.b1, mat.b2)
    y, s = oracle.ref_matmul(sub, x_bits, mat.dtype)
    return rows, y, s


# ------------------------------------------------------------- pack -------

@pytest.mark.parametrize("b1,b2", [(64, 64), (64, 128), (128, 128), (128, 256), (256, 64), (256, 256)])
@pytest.mark.parametrize("meta", ["idx2", "mask4"])
def test_pack_unpack_random(b1, b2, meta):
    dtype = "bf16" if b2 != 256 else "f16"
    note(f"pack random {b1}x{b2} {meta} {dtype}")
    w, tmap = random_case(b1 + b2, 3 * b1, 3 * b2, b1, b2, dtype)
    # sprinkle ties, signed zeros, subnormals, Inf and NaN
    rng = np.random.default_rng(1)
    for v in (0x8000, 0x0000, 0x0001, 0x8003, 0x7C00 if dtype == "f16" else 0x7F80, 0xFFC0):
        w[rng.random(w.shape) < 0.02] = v
    P = pack_gpu(w, tmap, b1, b2, dtype, meta)
    ref = oracle.pack(w, tmap, b1, b2, meta)
    got = streams(P)
    for key in ("dense", "val", "meta", "tidx"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    u = hb.tensor_to_bits(hb.unpack(P))
    np.testing.assert_array_equal(u, oracle.prune(w, tmap, b1, b2))


@pytest.mark.parametrize("config,index,meta", [(1, 0, "idx2"), (1, 0, "mask4"), (2, 0, "idx2"),
                                               (2, 0, "mask4"), (5, 0, "idx2"), (3, 1, "mask4")])
def test_pack_unpack_workloads(config, index, meta):
    mat, w, tmap = workload_matrix(config, index)
    note(f"pack workload {config}/{mat.name} {meta}")
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, meta)
    ref = oracle.pack(w, tmap, mat.b1, mat.b2, meta)
    got = streams(P)
    for key in ("dense", "val", "meta", "tidx"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    u = hb.tensor_to_bits(hb.unpack(P))
    np.testing.assert_array_equal(u, oracle.prune(w, tmap, mat.b1, mat.b2))


# ------------------------------------------------------------- GEMV -------

@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 11, 16])
@pytest.mark.parametrize("b1,b2,dtype,meta", [(64, 64, "bf16", "idx2"), (128, 128, "f16", "mask4"),
                                              (64, 256, "bf16", "mask4"), (256, 128, "bf16", "idx2")])
def test_gemv_random(m, b1, b2, dtype, meta):
    note(f"gemv random m={m} {b1}x{b2} {dtype} {meta}")
    torch = _torch()
    w, tmap = random_case(m * 7 + b2, 2 * b1, 5 * b2, b1, b2, dtype)
    x = wl.float32_to_bits(np.random.default_rng(m).standard_normal((m, 5 * b2)).astype(np.float32), dtype)
    P = pack_gpu(w, tmap, b1, b2, dtype, meta)
    y = hb.gemv(P, upload(x, dtype))
    torch.cuda.synchronize()
    yref, s = oracle.ref_matmul(oracle.prune(w, tmap, b1, b2), x, dtype)
    assert_close(y.cpu().numpy(), yref, s, what="gemv")


@pytest.mark.parametrize("config,index,m", [(1, 0, 1), (2, 0, 1), (2, 0, 4), (2, 0, 16)]
                         + [(3, i, m) for i in range(7) for m in (1, 4, 16)])
def test_gemv_workloads(config, index, m):
    """Every output of the 512x512 fp16 matrix, the 8B up projection (1, 4
    and 16 tokens) and all seven matrices of one 8B decoder layer at 1, 4
    and 16 tokens, against the oracle."""
    torch = _torch()
    mat, w, tmap = workload_matrix(config, index)
    note(f"gemv workload {config}/{mat.name} m={m}")
    x = mat.activation_bits(m)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    y = hb.gemv(P, upload(x, mat.dtype)).cpu().numpy()
    yref, s = oracle.ref_matmul(oracle.prune(w, tmap, mat.b1, mat.b2), x, mat.dtype)
    assert_close(y, yref, s, what=f"config {config} {mat.name} m={m}")


@pytest.mark.parametrize("index", range(6))
def test_gemv_70b_endpoints_full(index):
    """28672x8192 and 8192x28672 at 0%, 100% and checkerboard sparse tiles,
    full-size launch, every output against the oracle."""
    torch = _torch()
    mat = wl.workload(4).matrices[index]
    note(f"gemv 70B {mat.name}")
    w, tmap = mat.weight_bits(), mat.tile_map()
    x = mat.activation_bits(1)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    y = hb.gemv(P, upload(x, mat.dtype)).cpu().numpy()
    yref, s = oracle_full(w, tmap, mat.b1, mat.b2, x, mat.dtype)
    assert_close(y, yref, s, what=mat.name)
    expect = {"dense": 0, "sparse": tmap.size}.get(mat.name.split("_")[1], tmap.size // 2)
    assert P.layout.n_sparse == expect


@pytest.mark.parametrize("m", [1, 4, 16])
def test_gemv_grouped_layer(m):
    """One decoder layer's q, k, v and gate, up (same x, own tile maps and
    fractions) in one grouped launch: bitwise equal to separate launches,
    and every output within the bound of the oracle."""
    torch = _torch()
    W = wl.workload(3)
    mats = [mt for mt in W.matrices if mt.name in ("q", "k", "v", "gate", "up")]
    note(f"gemv grouped layer m={m}")
    x_bits = mats[0].activation_bits(m)
    xt = upload(x_bits, "bf16")
    Ps, refs = [], []
    for mt in mats:
        w = mt.weight_bits()
        tmap = mt.tile_map()
        Ps.append(pack_gpu(w, tmap, mt.b1, mt.b2, mt.dtype, "idx2"))
        refs.append((mt, w, tmap))
    outs = hb.gemv_grouped(Ps, xt)
    sep = [hb.gemv(P, xt) for P in Ps]
    torch.cuda.synchronize()
    for (mt, w, tmap), o, so in zip(refs, outs, sep):
        assert torch.equal(o, so), mt.name
        yref, sref = oracle_full(w, tmap, mt.b1, mt.b2, x_bits, mt.dtype)
        assert_close(o.cpu().numpy(), yref, sref, what=f"grouped {mt.name}")


def test_gemv_grouped_mixed_shapes():
    """Matrices of different b1 and n (one of them empty) in one launch, f16
    weights with mask4 codes and fp16 output, against separate launches and
    the oracle."""
    torch = _torch()
    note("gemv grouped mixed shapes")
    k, b2 = 384, 128
    specs = [(128, 64), (0, 128), (512, 256), (256, 128), (64, 64)]
    x_bits = wl.float32_to_bits(np.random.default_rng(9).standard_normal((3, k)).astype(np.float32), "f16")
    xt = upload(x_bits, "f16")
    Ps, refs = [], []
    for i, (n, b1) in enumerate(specs):
        w, tmap = random_case(40 + i, n, k, b1, b2, "f16")
        Ps.append(pack_gpu(w, tmap, b1, b2, "f16", "mask4"))
        refs.append((w, tmap, b1))
    outs = hb.gemv_grouped(Ps, xt, out_dtype=torch.float16)
    sep = [hb.gemv(P, xt, out_dtype=torch.float16) for P in Ps]
    torch.cuda.synchronize()
    for (w, tmap, b1), o, so in zip(refs, outs, sep):
        assert torch.equal(o, so)
        if w.shape[0] == 0:
            assert o.shape == (3, 0)
            continue
        yref, sref = oracle.ref_matmul(oracle.prune(w, tmap, b1, b2), x_bits, "f16")
        yb = oracle.widen(hb.tensor_to_bits(o), "f16")
        assert_close(yb, yref, sref, extra=np.abs(yref) * 2.0 ** -11 + 2.0 ** -25, what="grouped f16")


@pytest.mark.parametrize("rank", [8, 64, 256])
@pytest.mark.parametrize("m", [1, 3, 16])
@pytest.mark.parametrize("b1,b2,dtype,meta", [(128, 128, "bf16", "idx2"), (64, 256, "f16", "mask4")])
def test_gemv_lowrank(rank, m, b1, b2, dtype, meta):
    """Y = X W'^T + T U^T with T given: against the oracle, and bitwise
    equal to the plain decode product when U = 0."""
    torch = _torch()
    note(f"gemv lowrank r={rank} m={m} {b1}x{b2} {dtype} {meta}")
    n, k = 2 * b1, 2 * b2
    w, tmap = random_case(rank + m, n, k, b1, b2, dtype)
    rng = np.random.default_rng(rank * 31 + m)
    x = wl.float32_to_bits(rng.standard_normal((m, k)).astype(np.float32), dtype)
    t = (rng.standard_normal((m, rank)) * 4).astype(np.float32)
    u = wl.float32_to_bits(rng.standard_normal((n, rank)).astype(np.float32) * 0.05, dtype)
    P = pack_gpu(w, tmap, b1, b2, dtype, meta)
    xt = upload(x, dtype)
    tt = torch.from_numpy(t).to(dev())
    y = hb.gemv_lowrank(P, xt, tt, upload(u, dtype))
    y0 = hb.gemv_lowrank(P, xt, tt, upload(np.zeros_like(u), dtype))
    yg = hb.gemv(P, xt)
    torch.cuda.synchronize()
    assert torch.equal(y0, yg)
    yref, s = oracle.ref_lowrank(oracle.prune(w, tmap, b1, b2), x, t, u, dtype)
    assert_close(y.cpu().numpy(), yref, s, what="gemv lowrank")


@pytest.mark.parametrize("rem,m,b1,b2,dtype,meta", [(4, 1, 64, 128, "bf16", "idx2"),
                                                    (64, 2, 64, 256, "f16", "mask4"),
                                                    (128, 1, 128, 128, "bf16", "idx2"),
                                                    (132, 2, 64, 64, "bf16", "mask8"),
                                                    (64, 4, 64, 128, "bf16", "idx2"),
                                                    (128, 3, 128, 256, "f16", "mask4")])
def test_gemv_half_slab_last_round(rem, m, b1, b2, dtype, meta):
    """Decode over 2 C + rem slabs (C = the device's compute units): where
    2 rem <= C (and the mixed launch fits on the CUs at once) the last
    round's slabs run as 8-row halves.  Bitwise equal to
    the grouped launch (whole slabs only), the low-rank entry point with
    U = 0 bitwise equal too, and both products against the oracle."""
    torch = _torch()
    n, k, rank = (2 * device_cus() + rem) * 16, 1024, 16
    note(f"gemv half slabs n={n} m={m} {b1}x{b2} {dtype} {meta}")
    w, tmap = random_case(rem * 7 + m, n, k, b1, b2, dtype)
    rng = np.random.default_rng(rem + 100 * m)
    x = wl.float32_to_bits(rng.standard_normal((m, k)).astype(np.float32), dtype)
    t = (rng.standard_normal((m, rank)) * 4).astype(np.float32)
    u = wl.float32_to_bits(rng.standard_normal((n, rank)).astype(np.float32) * 0.05, dtype)
    P = pack_gpu(w, tmap, b1, b2, dtype, meta)
    xt, tt = upload(x, dtype), torch.from_numpy(t).to(dev())
    y = hb.gemv(P, xt)
    (yg,) = hb.gemv_grouped([P], xt)
    y0 = hb.gemv_lowrank(P, xt, tt, upload(np.zeros_like(u), dtype))
    yl = hb.gemv_lowrank(P, xt, tt, upload(u, dtype))
    torch.cuda.synchronize()
    assert torch.equal(y, yg)
    assert torch.equal(y0, yg)
    yref, s = oracle_full(w, tmap, b1, b2, x, dtype, meta=meta)
    assert_close(y.cpu().numpy(), yref, s, what="gemv half slabs")
    lref, ls = oracle_full_lowrank(w, tmap, b1, b2, x, t, u, dtype, meta=meta)
    assert_close(yl.cpu().numpy(), lref, ls, what="gemv lowrank half slabs")


_CAPTURE_FIRST = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
from matmul_pack_b1_amd import binding as hb
from matmul_pack_b1_amd import workloads as wl
cus = torch.cuda.get_device_properties(0).multi_processor_count
n, k, b1, b2 = (2 * cus + 96) * 16, 2048, 64, 256
rng = np.random.default_rng(5)
w_bits = wl.float32_to_bits(rng.standard_normal((n, k)).astype(np.float32) * 0.02, "f16")
tmap = (rng.random((n // b1, k // b2)) < 0.6).astype(np.uint8)
dev = torch.device("cuda:0")
w = torch.from_numpy(w_bits.view(np.int16)).to(dev).view(torch.float16)
P = hb.pack(w, tmap, b1, b2, "mask8")
x = torch.from_numpy(rng.standard_normal((1, k)).astype(np.float32)).to(dev).half()
out = torch.empty(1, n, device=dev)
torch.cuda.synchronize()
s = torch.cuda.Stream()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=s):
    hb.gemv(P, x, out=out)
reps = []
for _ in range(3):
    g.replay()
    torch.cuda.synchronize()
    reps.append(out.clone())
    out.zero_()
    torch.cuda.synchronize()
ye = hb.gemv(P, x)
torch.cuda.synchronize()
assert all(torch.equal(r, ye) for r in reps), "replay differs from the eager product"
assert bool(torch.isfinite(ye).all())
print("capture-first ok", flush=True)
"""


def test_gemv_mixed_launch_first_call_under_capture():
    """The mixed decode launch looks up its occupancy on its first call; in a
    fresh process that first call is made under graph capture (fp16 weights,
    mask8 codes, b2 = 256, 2 C + 96 slabs).  Three replays, with eager work
    between them, equal the eager product bitwise."""
    import os
    import subprocess
    note("gemv mixed launch, first call under graph capture (subprocess)")
    repo = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _CAPTURE_FIRST, repo], capture_output=True, text=True, timeout=110)
    assert r.returncode == 0 and "capture-first ok" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("rank,k,m,dtype", [(64, 4096, 1, "bf16"), (64, 4096, 16, "bf16"), (1, 72, 3, "f16"),
                                             (256, 5120, 40, "bf16"), (8, 2056, 17, "f16"), (20, 5120, 300, "bf16"),
                                             (64, 1024, 2048, "f16")])
def test_lowrank_project(rank, k, m, dtype):
    """T = X V (V held transposed, rank x k) against the oracle's product,
    over token blocks of 16 with a ragged last block and K tails that do
    not fill a stride of 2048; bitwise repeatable."""
    torch = _torch()
    note(f"lowrank project r={rank} k={k} m={m} {dtype}")
    rng = np.random.default_rng(rank + k + m)
    v = wl.float32_to_bits(rng.standard_normal((rank, k)).astype(np.float32) * 0.05, dtype)
    x = wl.float32_to_bits(rng.standard_normal((m, k)).astype(np.float32), dtype)
    vt, xt = upload(v, dtype), upload(x, dtype)
    t = hb.lowrank_project(vt, xt)
    t2 = hb.lowrank_project(vt, xt)
    torch.cuda.synchronize()
    assert torch.equal(t, t2)
    tref, s = oracle.ref_matmul(v, x, dtype)
    assert_close(t.cpu().numpy(), tref, s, what="lowrank project")


def test_lowrank_project_strided_and_empty():
    """Row strides above k for v, x and t; k = 0 gives T = 0."""
    torch = _torch()
    note("lowrank project strided / k = 0")
    rng = np.random.default_rng(5)
    rank, k, m = 24, 256, 5
    v = wl.float32_to_bits(rng.standard_normal((rank, k + 40)).astype(np.float32), "bf16")
    x = wl.float32_to_bits(rng.standard_normal((m, k + 16)).astype(np.float32), "bf16")
    tbuf = torch.full((m, rank + 8), 7.0, dtype=torch.float32, device=dev())
    hb.lowrank_project(upload(v, "bf16")[:, :k], upload(x, "bf16")[:, :k], out=tbuf[:, :rank])
    got = tbuf.cpu().numpy()
    tref, s = oracle.ref_matmul(v[:, :k], x[:, :k], "bf16")
    assert_close(got[:, :rank], tref, s, what="strided project")
    assert (got[:, rank:] == 7.0).all()
    z = hb.lowrank_project(torch.empty((rank, 0), dtype=torch.bfloat16, device=dev()),
                           torch.empty((m, 0), dtype=torch.bfloat16, device=dev()))
    assert z.shape == (m, rank) and (z.cpu() == 0).all()


def test_sparse_lowrank_end_to_end():
    """Two launches on the 8B up projection shape: T = X V with the
    projection kernel, then the hybrid product with T U^T added (2:4 sparse +
    rank 64).  The oracle computes T itself; its error bound adds T's own
    bound carried through |U|."""
    torch = _torch()
    note("sparse + low-rank end to end")
    mat, w, tmap = workload_matrix(2, 0)
    rank, m = 64, 4
    rng = np.random.default_rng(64)
    v = wl.float32_to_bits(rng.standard_normal((rank, mat.k)).astype(np.float32) * 0.02, "bf16")
    u = wl.float32_to_bits(rng.standard_normal((mat.n, rank)).astype(np.float32) * 0.02, "bf16")
    x = mat.activation_bits(m)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    y = hb.sparse_lowrank_gemv(P, upload(v, "bf16"), upload(u, "bf16"), upload(x, "bf16")).cpu().numpy()
    t_ref, s_t = oracle.ref_matmul(v, x, "bf16")
    yref, s = oracle_full_lowrank(w, tmap, mat.b1, mat.b2, x, t_ref, u, "bf16")
    extra = REL * (s_t @ np.abs(oracle.widen(u, "bf16")).T)
    assert_close(y, yref, s, extra=extra, what="sparse + low-rank")


@pytest.mark.parametrize("m,rank,dtype", [(9, 64, "bf16"), (40, 8, "f16"), (130, 256, "bf16"), (300, 64, "f16")])
def test_gemm_lowrank(m, rank, dtype):
    """Prefill sizes: the matrix-core product with the T U^T epilogue against
    the oracle (ragged token tiles); rank 0 and U = 0 give the plain product
    bitwise."""
    torch = _torch()
    note(f"gemm lowrank m={m} r={rank} {dtype}")
    b1, b2 = 64, 128
    n, k = 5 * b1, 3 * b2
    w, tmap = random_case(m + rank, n, k, b1, b2, dtype)
    rng = np.random.default_rng(m * 3 + rank)
    x = wl.float32_to_bits(rng.standard_normal((m, k)).astype(np.float32), dtype)
    t = (rng.standard_normal((m, rank)) * 4).astype(np.float32)
    u = wl.float32_to_bits(rng.standard_normal((n, rank)).astype(np.float32) * 0.05, dtype)
    P = pack_gpu(w, tmap, b1, b2, dtype, "idx2")
    xt, tt = upload(x, dtype), torch.from_numpy(t).to(dev())
    y = hb.gemm_lowrank(P, xt, tt, upload(u, dtype))
    y0 = hb.gemm_lowrank(P, xt, tt, upload(np.zeros_like(u), dtype))
    yr0 = hb.gemm_lowrank(P, xt, tt[:, :0], upload(u, dtype)[:, :0])
    yg = hb.gemm(P, xt)
    torch.cuda.synchronize()
    assert torch.equal(y0, yg) and torch.equal(yr0, yg)
    yref, s = oracle.ref_lowrank(oracle.prune(w, tmap, b1, b2), x, t, u, dtype)
    assert_close(y.cpu().numpy(), yref, s, what="gemm lowrank")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_gemm_lowrank_lds_shape(dtype):
    """The LDS-fed kernel's T U^T epilogue in both weight dtypes (bf16: T as
    hi + lo bf16 products; fp16: fp32 16x16x4 products): 8192 rows at 1024
    tokens run the 128-token LDS shape on a 256-CU device (the small
    matrices of test_gemm_lowrank take the register-fed kernel).  Sampled
    tile rows against the oracle; U = 0 gives the plain product bitwise."""
    torch = _torch()
    note(f"gemm lowrank lds shape {dtype}")
    b1, b2, n, k, m, rank = 64, 128, 8192, 256, 1024, 64
    w, tmap = random_case(8192 + rank, n, k, b1, b2, dtype)
    rng = np.random.default_rng(1024 + rank)
    x = wl.float32_to_bits(rng.standard_normal((m, k)).astype(np.float32), dtype)
    t = (rng.standard_normal((m, rank)) * 4).astype(np.float32)
    u = wl.float32_to_bits(rng.standard_normal((n, rank)).astype(np.float32) * 0.05, dtype)
    P = pack_gpu(w, tmap, b1, b2, dtype, "idx2")
    xt, tt = upload(x, dtype), torch.from_numpy(t).to(dev())
    y = hb.gemm_lowrank(P, xt, tt, upload(u, dtype))
    y0 = hb.gemm_lowrank(P, xt, tt, upload(np.zeros_like(u), dtype))
    yg = hb.gemm(P, xt)
    torch.cuda.synchronize()
    assert torch.equal(y0, yg)
    tile_rows = np.sort(np.random.default_rng(7).choice(n // b1, size=3, replace=False))
    rows = np.concatenate([np.arange(tr * b1, (tr + 1) * b1) for tr in tile_rows])
    yref, s = oracle.ref_lowrank(oracle.prune(w[rows], tmap[tile_rows], b1, b2), x, t, u[rows], dtype)
    assert_close(y.cpu().numpy()[:, rows], yref, s, what="gemm lowrank lds shape")


def test_gemm_lowrank_small_m_and_strides():
    """Up to the crossover (8 tokens on this 256-row matrix) the fused decode
    kernel runs (bitwise the decode entry point); above, a y with a row
    stride larger than n keeps its padding."""
    torch = _torch()
    note("gemm lowrank m <= 8 and strided y")
    b1, b2, n, k, rank = 128, 128, 256, 512, 32
    w, tmap = random_case(31, n, k, b1, b2, "bf16")
    rng = np.random.default_rng(31)
    u = upload(wl.float32_to_bits(rng.standard_normal((n, rank)).astype(np.float32) * 0.05, "bf16"), "bf16")
    P = pack_gpu(w, tmap, b1, b2, "bf16", "idx2")
    for m in (1, 8):
        x = upload(wl.float32_to_bits(rng.standard_normal((m, k)).astype(np.float32), "bf16"), "bf16")
        t = torch.randn((m, rank), device=dev())
        assert torch.equal(hb.gemm_lowrank(P, x, t, u), hb.gemv_lowrank(P, x, t, u))
    m = 70
    xb = wl.float32_to_bits(rng.standard_normal((m, k)).astype(np.float32), "bf16")
    tb = rng.standard_normal((m, rank)).astype(np.float32)
    ybig = torch.full((m, n + 36), 3.0, device=dev())
    hb.gemm_lowrank(P, upload(xb, "bf16"), torch.from_numpy(tb).to(dev()), u, out=ybig[:, :n])
    torch.cuda.synchronize()
    assert torch.all(ybig[:, n:] == 3.0)
    yref, s = oracle.ref_lowrank(oracle.prune(w, tmap, b1, b2), xb, tb, hb.tensor_to_bits(u), "bf16")
    assert_close(ybig[:, :n].cpu().numpy(), yref, s, what="strided gemm lowrank")


@pytest.mark.parametrize("m", [12, 40, 100, 256])
def test_sparse_lowrank_prefill_qwen14b(m):
    """17408 x 5120 (64 x 64 tiles, 60% 2:4) + rank 64: the projection on
    the matrix cores (above 16 tokens) and the matrix-core product with the
    T U^T epilogue, through each kernel variant (register-fed with one row
    group at 12 tokens and two at 40, the LDS-fed kernel's 64-token shape at
    100 and its larger shapes at 256), every output against the oracle; the
    oracle computes T itself and the bound carries T's own error through
    |U|."""
    torch = _torch()
    note(f"sparse + low-rank prefill qwen14b m={m}")
    mat, w, tmap = workload_matrix(5, 0)
    rank = 64
    rng = np.random.default_rng(65)
    v = wl.float32_to_bits(rng.standard_normal((rank, mat.k)).astype(np.float32) * 0.02, "bf16")
    u = wl.float32_to_bits(rng.standard_normal((mat.n, rank)).astype(np.float32) * 0.02, "bf16")
    x = mat.activation_bits(m)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    y = hb.sparse_lowrank_gemm(P, upload(v, "bf16"), upload(u, "bf16"), upload(x, "bf16")).cpu().numpy()
    t_ref, s_t = oracle.ref_matmul(v, x, "bf16")
    yref, s = oracle_full_lowrank(w, tmap, mat.b1, mat.b2, x, t_ref, u, "bf16")
    extra = REL * (s_t @ np.abs(oracle.widen(u, "bf16")).T)
    assert_close(y, yref, s, extra=extra, what="prefill sparse + low-rank")


def test_sparse_lowrank_prefill_tall():
    """8192 x 28672 (128 x 128 tiles, checkerboard) + rank 32 at 200 tokens:
    the register-fed product above 128 tokens (the shape a short, deep
    matrix takes there) with its T U^T epilogue; every output against the
    oracle."""
    torch = _torch()
    note("sparse + low-rank prefill 70b tall m=200")
    mat, w, tmap = workload_matrix(4, 5)
    rank, m = 32, 200
    rng = np.random.default_rng(200)
    v = wl.float32_to_bits(rng.standard_normal((rank, mat.k)).astype(np.float32) * 0.01, "bf16")
    u = wl.float32_to_bits(rng.standard_normal((mat.n, rank)).astype(np.float32) * 0.02, "bf16")
    x = mat.activation_bits(m)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    y = hb.sparse_lowrank_gemm(P, upload(v, "bf16"), upload(u, "bf16"), upload(x, "bf16")).cpu().numpy()
    t_ref, s_t = oracle.ref_matmul(v, x, "bf16")
    yref, s = oracle_full_lowrank(w, tmap, mat.b1, mat.b2, x, t_ref, u, "bf16")
    extra = REL * (s_t @ np.abs(oracle.widen(u, "bf16")).T)
    assert_close(y, yref, s, extra=extra, what="tall prefill sparse + low-rank")


def test_gemm_lowrank_output_16bit():
    """A 16-bit y is rounded once, after the low-rank term is added."""
    torch = _torch()
    note("gemm lowrank bf16 out")
    w, tmap = random_case(41, 256, 512, 128, 128, "bf16")
    rng = np.random.default_rng(41)
    x = wl.float32_to_bits(rng.standard_normal((96, 512)).astype(np.float32), "bf16")
    t = rng.standard_normal((96, 64)).astype(np.float32)
    u = wl.float32_to_bits(rng.standard_normal((256, 64)).astype(np.float32) * 0.05, "bf16")
    P = pack_gpu(w, tmap, 128, 128, "bf16", "idx2")
    y = hb.gemm_lowrank(P, upload(x, "bf16"), torch.from_numpy(t).to(dev()), upload(u, "bf16"),
                        out_dtype=torch.bfloat16)
    yb = oracle.widen(hb.tensor_to_bits(y), "bf16")
    yref, s = oracle.ref_lowrank(oracle.prune(w, tmap, 128, 128), x, t, u, "bf16")
    assert_close(yb, yref, s, extra=np.abs(yref) * 2.0 ** -8 + 2.0 ** -133, what="bf16 out low-rank")


def test_gemv_output_16bit():
    torch = _torch()
    mat, w, tmap = workload_matrix(2, 0)
    note("gemv bf16 output")
    x = mat.activation_bits(3)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    y = hb.gemv(P, upload(x, "bf16"), out_dtype=torch.bfloat16)
    yb = oracle.widen(hb.tensor_to_bits(y), "bf16")
    yref, s = oracle.ref_matmul(oracle.prune(w, tmap, mat.b1, mat.b2), x, "bf16")
    half_ulp = np.abs(yref) * 2.0 ** -8 + 1e-30
    assert_close(yb, yref, s, extra=half_ulp, what="bf16 out")


@pytest.mark.parametrize("m", [1, 16])
def test_gemv_grouped_max_count(m):
    """HYB_MAX_GROUP matrices in one call, short ones (8 or 16 wavefronts
    per slab) mixed with tall ones (4): bitwise equal to separate launches
    and within the oracle's bound on every matrix."""
    torch = _torch()
    note(f"gemv grouped x{hb.MAX_GROUP} m={m}")
    k = 512
    rng = np.random.default_rng(160 + m)
    x = wl.float32_to_bits(rng.standard_normal((m, k)).astype(np.float32), "bf16")
    xt = upload(x, "bf16")
    Ps, refs = [], []
    for i in range(hb.MAX_GROUP):
        n = 128 * (1 + i % 3) if i % 2 else 8192
        w, tmap = random_case(1600 + i, n, k, 128, 128, "bf16", frac=0.2 + 0.04 * i)
        Ps.append(pack_gpu(w, tmap, 128, 128, "bf16", "idx2"))
        refs.append((w, tmap))
    outs = hb.gemv_grouped(Ps, xt)
    sep = [hb.gemv(P, xt) for P in Ps]
    torch.cuda.synchronize()
    for i, ((w, tmap), o, so) in enumerate(zip(refs, outs, sep)):
        assert torch.equal(o, so), i
        yref, sref = oracle_full(w, tmap, 128, 128, x, "bf16")
        assert_close(o.cpu().numpy(), yref, sref, what=f"grouped matrix {i}")


# ------------------------------------------------------------- GEMM -------

@pytest.mark.parametrize("m", [17, 33, 64, 100, 130, 257])
@pytest.mark.parametrize("b1,b2,dtype,meta", [(64, 64, "bf16", "idx2"), (128, 128, "f16", "mask4"),
                                              (256, 256, "bf16", "mask4"), (64, 128, "bf16", "idx2")])
def test_gemm_random(m, b1, b2, dtype, meta):
    note(f"gemm random m={m} {b1}x{b2} {dtype} {meta}")
    torch = _torch()
    n = 3 * b1 if b1 == 64 else 2 * b1   # 192 rows exercises a half-empty 128-row block
    k = 3 * b2
    w, tmap = random_case(m + b1, n, k, b1, b2, dtype)
    x = wl.float32_to_bits(np.random.default_rng(m).standard_normal((m, k)).astype(np.float32), dtype)
    P = pack_gpu(w, tmap, b1, b2, dtype, meta)
    y = hb.gemm(P, upload(x, dtype))
    torch.cuda.synchronize()
    yref, s = oracle.ref_matmul(oracle.prune(w, tmap, b1, b2), x, dtype)
    assert_close(y.cpu().numpy(), yref, s, what="gemm")


def random_rows_check(w, tmap, b1, b2, x, y, dtype, seed, meta="idx2", count=3):
    """Oracle check of `count` sampled tile rows of a random case."""
    tile_rows = np.sort(np.random.default_rng(seed).choice(tmap.shape[0], size=count, replace=False))
    rows = np.concatenate([np.arange(t * b1, (t + 1) * b1) for t in tile_rows])
    yref, s = oracle.ref_matmul(oracle.prune(w[rows], tmap[tile_rows], b1, b2, meta), x, dtype)
    assert_close(y[:, rows], yref, s, what=f"sampled rows {tile_rows.tolist()}")


@pytest.mark.parametrize("n,m", [(8192, 1024), (8192, 2048), (16384, 256)])
@pytest.mark.parametrize("b1,b2,dtype,meta", [(64, 64, "bf16", "idx2"), (128, 128, "f16", "mask4"),
                                              (256, 256, "bf16", "mask4"), (64, 128, "bf16", "idx2")])
def test_gemm_lds_shapes_random(n, m, b1, b2, dtype, meta):
    """Matrices with enough 256-row blocks that the launcher runs an LDS-fed
    shape on a 256-CU device: 8192 rows at 1024 tokens (the 128-token
    shape), 8192 rows at 2048 (the 256-token shape) and 16384 rows at 256
    (the 64-token shape), in every tile size, dtype and metadata kind of
    test_gemm_random (whose small matrices take the register-fed kernel at
    every token count); every output against the oracle."""
    torch = _torch()
    note(f"gemm lds shapes n={n} m={m} {b1}x{b2} {dtype} {meta}")
    k = 2 * b2
    w, tmap = random_case(n + m + b2, n, k, b1, b2, dtype)
    x = wl.float32_to_bits(np.random.default_rng(m + n).standard_normal((m, k)).astype(np.float32), dtype)
    P = pack_gpu(w, tmap, b1, b2, dtype, meta)
    expect_route(P, m, "lds", token_blocks={1024: 8, 2048: 16, 256: 4}[m])
    y = hb.gemm(P, upload(x, dtype)).cpu().numpy()
    yref, s = oracle_full(w, tmap, b1, b2, x, dtype)
    assert_close(y, yref, s, what=f"gemm lds n={n} m={m}")


@pytest.mark.parametrize("config,index,m,route", [(3, 1, 384, ("register", 2, 8, 1)),
                                                  (3, 0, 160, ("register", 2, 4, 2)),
                                                  (3, 6, 256, ("split", 16, 8, 4))])
def test_gemm_small_matrices_above_128(config, index, m, route):
    """Few 256-row blocks above 128 tokens: the launcher prices every
    register-fed shape, plain and split, against the LDS shapes and, on a
    256-CU device, runs 32 tokens x 64 rows on eight wavefronts for the 1024
    x 4096 k projection at 384 tokens, 32 tokens x 128 rows on four
    wavefronts for the 4096-row q projection at 160 tokens (ragged), and the
    LDS-fed 256-token x 256-row tile with K cut into 14 parts for the 4096 x
    14336 down projection at 256 tokens.  Every output against the
    oracle."""
    torch = _torch()
    mat, w, tmap = workload_matrix(config, index)
    note(f"gemm small matrix {mat.name} m={m}")
    x = mat.activation_bits(m)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    expect_route(P, m, *route)
    yref, s = oracle_full(w, tmap, mat.b1, mat.b2, x, mat.dtype)
    y = hb.gemm(P, upload(x, mat.dtype)).cpu().numpy()
    assert_close(y, yref, s, what=f"gemm {mat.name} m={m}")


@pytest.mark.parametrize("m", [8, 16, 64, 128, 256, 2048])
def test_gemm_qwen14b_full(m):
    """17408x5120, 64x64 tiles, 60% sparse tiles; M from 8 to 2048 through
    hyb_gemm and through the matrix-core entry point, every output against
    the oracle.  At 2048 tokens a 256-CU device runs two whole rounds of
    256-token tiles (the first 64 of 68 row blocks) and the last 4 row
    blocks' 32 tiles with K cut into 5 parts."""
    torch = _torch()
    mat, w, tmap = workload_matrix(5, 0)
    note(f"gemm qwen14b m={m}")
    x = mat.activation_bits(m)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    if m == 2048:
        expect_route(P, m, "split", 16, 8, 4)
        assert hb.workspace_bytes(P, m) == 32 * 5 * 256 * 256 * 4
    xt = upload(x, mat.dtype)
    yref, s = oracle_full(w, tmap, mat.b1, mat.b2, x, mat.dtype)
    y = hb.gemm(P, xt).cpu().numpy()
    assert_close(y, yref, s, what=f"gemm m={m}")
    y2 = hb.gemm_mfma(P, xt).cpu().numpy()
    assert_close(y2, yref, s, what=f"gemm_mfma m={m}")


@pytest.mark.parametrize("m,route", [(160, ("split", 12, 8, 4)), (200, ("split", 16, 8, 4)), (256, ("split", 16, 8, 4)),
                                     (300, ("lds", 8, 8, 4)), (512, ("lds", 8, 8, 4)), (700, ("lds", 12, 8, 4)),
                                     (1024, ("lds", 16, 8, 4))])
def test_gemm_8b_up_shapes(m, route):
    """14336x4096, 128x128 tiles, 70% sparse tiles.  From 129 tokens the
    launcher picks among the 256-row LDS tiles (256, 192, 128 or 64 tokens
    per workgroup); on a 256-CU device these token counts select the
    192-token tile with K cut into 4 parts (160, ragged), the 256-token tile
    with K cut into 2 parts (200 ragged, 256), and one round of plain tiles:
    128 tokens (300 ragged, 512), 192 (700 ragged) and 256 (1024).  Every
    output against the oracle."""
    torch = _torch()
    mat, w, tmap = workload_matrix(2, 0)
    note(f"gemm 8b up m={m}")
    x = mat.activation_bits(m)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    expect_route(P, m, *route)
    yref, s = oracle_full(w, tmap, mat.b1, mat.b2, x, mat.dtype)
    y = hb.gemm(P, upload(x, mat.dtype)).cpu().numpy()
    assert_close(y, yref, s, what=f"gemm m={m}")


@pytest.mark.parametrize("m,route", [(64, ("split", 4, 4, 2)), (160, ("split", 12, 8, 4)),
                                     (256, ("split", 16, 8, 4)), (512, ("split", 16, 8, 4))])
def test_gemm_tall_70b(m, route):
    """8192x28672 (32 blocks of 256 rows), 128x128 tiles in a checkerboard:
    up to a few hundred tokens every plain LDS shape leaves most CUs of a
    256-CU device idle.  At 64 tokens the launcher runs the register-fed
    shape (128 rows by 64 tokens, K split over four wavefronts and across
    256 workgroups); at 160 (ragged) the 192-token LDS tile, at 256 and 512
    the 256-token one (1 and 2 token blocks), each with K cut into 8 or 4
    equal parts over 256 workgroups.  Every output against the oracle."""
    torch = _torch()
    mat, w, tmap = workload_matrix(4, 5)
    note(f"gemm 70b tall m={m}")
    x = mat.activation_bits(m)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    expect_route(P, m, *route)
    yref, s = oracle_full(w, tmap, mat.b1, mat.b2, x, mat.dtype)
    y = hb.gemm(P, upload(x, mat.dtype)).cpu().numpy()
    assert_close(y, yref, s, what=f"gemm tall m={m}")


@pytest.mark.parametrize("m,route", [(80, ("split", 3, 4, 2)), (128, ("split", 8, 8, 4))])
def test_gemm_wide_70b(m, route):
    """28672x8192 (128x128 tiles, checkerboard): at 80 tokens (ragged) the
    launcher splits 48-token x 128-row tiles over 256 workgroups; at 128 it
    splits the 112 tiles of the LDS-fed 128-token x 256-row shape over 256
    workgroups.  Every output against the oracle."""
    torch = _torch()
    mat, w, tmap = workload_matrix(4, 2)
    note(f"gemm 70b wide m={m}")
    x = mat.activation_bits(m)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    expect_route(P, m, *route)
    yref, s = oracle_full(w, tmap, mat.b1, mat.b2, x, mat.dtype)
    y = hb.gemm(P, upload(x, mat.dtype)).cpu().numpy()
    assert_close(y, yref, s, what=f"gemm wide m={m}")


@pytest.mark.parametrize("m", [20, 64])
def test_gemm_two_row_groups_odd(m):
    """16448 rows (257 row groups of 64, more than one round on a 256-CU
    device): from 17 tokens the register-fed kernel takes two row groups per
    workgroup, and the last workgroup's second group lies past the last row."""
    torch = _torch()
    note(f"gemm two row groups, odd count, m={m}")
    n, k, b1, b2 = 64 * 257, 192, 64, 64
    w, tmap = random_case(77 + m, n, k, b1, b2, "bf16", frac=0.6)
    x = wl.float32_to_bits(np.random.default_rng(m).standard_normal((m, k)).astype(np.float32), "bf16")
    P = pack_gpu(w, tmap, b1, b2, "bf16", "idx2")
    y = hb.gemm(P, upload(x, "bf16"))
    torch.cuda.synchronize()
    yref, s = oracle.ref_matmul(oracle.prune(w, tmap, b1, b2), x, "bf16")
    assert_close(y.cpu().numpy(), yref, s, what="gemm two row groups")


def test_gemm_4096_tokens_full():
    """4096 tokens (16 token blocks of the 256-token LDS shape) on a 1024 x
    1024 matrix, every output against the oracle."""
    torch = _torch()
    note("gemm m=4096 full")
    w, tmap = random_case(4096, 1024, 1024, 64, 128, "bf16")
    x = wl.float32_to_bits(np.random.default_rng(4096).standard_normal((4096, 1024)).astype(np.float32), "bf16")
    P = pack_gpu(w, tmap, 64, 128, "bf16", "idx2")
    y = hb.gemm(P, upload(x, "bf16"))
    torch.cuda.synchronize()
    yref, s = oracle.ref_matmul(oracle.prune(w, tmap, 64, 128), x, "bf16")
    assert_close(y.cpu().numpy(), yref, s, what="gemm m=4096")


def test_gemm_output_16bit():
    torch = _torch()
    note("gemm fp16 output")
    w, tmap = random_case(3, 256, 512, 128, 128, "f16")
    x = wl.float32_to_bits(np.random.default_rng(3).standard_normal((96, 512)).astype(np.float32), "f16")
    P = pack_gpu(w, tmap, 128, 128, "f16", "idx2")
    y = hb.gemm(P, upload(x, "f16"), out_dtype=torch.float16)
    yb = oracle.widen(hb.tensor_to_bits(y), "f16")
    yref, s = oracle.ref_matmul(oracle.prune(w, tmap, 128, 128), x, "f16")
    assert_close(yb, yref, s, extra=np.abs(yref) * 2.0 ** -11 + 2.0 ** -25, what="f16 out")


# ------------------------------------------------------- exact pins -------

@pytest.mark.parametrize("kernel", ["gemv", "gemm_mfma"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_one_hot_columns_exact(kernel, dtype):
    """x = e_c gives column c of W' bit for bit (subnormals included)."""
    torch = _torch()
    note(f"one-hot {kernel} {dtype}")
    b1, b2 = 64, 128
    w, tmap = random_case(11, 2 * b1, 2 * b2, b1, b2, dtype)
    w[::7, ::5] = 0x0001   # smallest subnormal
    cols = np.array([0, 1, 63, 64, 100, 127, 128, 255])
    one = 0x3F80 if dtype == "bf16" else 0x3C00
    m = len(cols) if kernel == "gemv" else 32
    x = np.zeros((m, 2 * b2), np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = one
    P = pack_gpu(w, tmap, b1, b2, dtype, "mask4")
    fn = hb.gemv if kernel == "gemv" else hb.gemm_mfma
    y = fn(P, upload(x, dtype)).cpu().numpy()
    wp = oracle.prune(w, tmap, b1, b2)
    for i, c in enumerate(cols):
        np.testing.assert_array_equal(y[i], oracle.widen(wp[:, c], dtype).astype(np.float32))
    assert np.all(y[len(cols):] == 0)


@pytest.mark.parametrize("kernel", ["gemv", "gemm_mfma"])
def test_small_integers_exact(kernel):
    torch = _torch()
    note(f"integers {kernel}")
    rng = np.random.default_rng(12)
    b1, b2 = 128, 64
    n, k, m = 256, 640, (5 if kernel == "gemv" else 70)
    w = wl.float32_to_bits(rng.integers(-3, 4, size=(n, k)).astype(np.float32), "bf16")
    x = wl.float32_to_bits(rng.integers(-3, 4, size=(m, k)).astype(np.float32), "bf16")
    tmap = (rng.random((n // b1, k // b2)) < 0.5).astype(np.uint8)
    P = pack_gpu(w, tmap, b1, b2, "bf16", "idx2")
    fn = hb.gemv if kernel == "gemv" else hb.gemm_mfma
    y = fn(P, upload(x, "bf16")).cpu().numpy()
    yref, _ = oracle.ref_matmul(oracle.prune(w, tmap, b1, b2), x, "bf16")
    np.testing.assert_array_equal(y.astype(np.float64), yref)


@pytest.mark.parametrize("kernel", ["gemv", "gemm_mfma"])
def test_zero_input_gives_plus_zero(kernel):
    torch = _torch()
    note(f"zero input {kernel}")
    w, tmap = random_case(13, 128, 256, 64, 128, "bf16")
    P = pack_gpu(w, tmap, 64, 128, "bf16", "idx2")
    x = torch.zeros((4 if kernel == "gemv" else 40, 256), dtype=torch.bfloat16, device=dev())
    fn = hb.gemv if kernel == "gemv" else hb.gemm_mfma
    y = fn(P, x).cpu().numpy()
    assert np.all(y == 0) and not np.any(np.signbit(y))


# ------------------------------------------------------------ edges -------

def test_empty_and_degenerate():
    torch = _torch()
    note("edges")
    # k = 0: no tiles along K, the product is an empty sum
    P = pack_gpu(np.zeros((128, 0), np.uint16), np.zeros((2, 0), np.uint8), 64, 64, "bf16", "idx2")
    x = torch.zeros((3, 0), dtype=torch.bfloat16, device=dev())
    y = torch.full((3, 128), 7.0, device=dev())
    hb.gemv(P, x, out=y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)
    y = torch.full((40, 128), 7.0, device=dev())
    hb.gemm_mfma(P, torch.zeros((40, 0), dtype=torch.bfloat16, device=dev()), out=y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)
    # m = 0 leaves y untouched
    w, tmap = random_case(14, 64, 64, 64, 64, "bf16")
    P = pack_gpu(w, tmap, 64, 64, "bf16", "idx2")
    y = torch.full((0, 64), 1.0, device=dev())
    hb.gemv(P, torch.zeros((0, 64), dtype=torch.bfloat16, device=dev()), out=y)
    # n = 0
    P0 = pack_gpu(np.zeros((0, 128), np.uint16), np.zeros((0, 2), np.uint8), 64, 64, "bf16", "idx2")
    hb.gemv(P0, torch.zeros((2, 128), dtype=torch.bfloat16, device=dev()))
    # all-dense and all-sparse maps
    for val in (0, 1):
        w, _ = random_case(15, 128, 256, 64, 128, "bf16")
        tmap = np.full((2, 2), val, np.uint8)
        P = pack_gpu(w, tmap, 64, 128, "bf16", "idx2")
        x = wl.float32_to_bits(np.random.default_rng(val).standard_normal((2, 256)).astype(np.float32), "bf16")
        y = hb.gemv(P, upload(x, "bf16")).cpu().numpy()
        yref, s = oracle.ref_matmul(oracle.prune(w, tmap, 64, 128), x, "bf16")
        assert_close(y, yref, s, what=f"map={val}")
    torch.cuda.synchronize()


def test_strided_rows():
    """x and y with row strides larger than their widths."""
    torch = _torch()
    note("strides")
    w, tmap = random_case(16, 128, 256, 64, 128, "bf16")
    P = pack_gpu(w, tmap, 64, 128, "bf16", "idx2")
    x = wl.float32_to_bits(np.random.default_rng(2).standard_normal((3, 256)).astype(np.float32), "bf16")
    xbig = torch.zeros((3, 264), dtype=torch.bfloat16, device=dev())
    xbig[:, :256] = upload(x, "bf16")
    ybig = torch.full((3, 200), 5.0, device=dev())
    hb.gemv(P, xbig[:, :256], out=ybig[:, :128])
    torch.cuda.synchronize()
    yref, s = oracle.ref_matmul(oracle.prune(w, tmap, 64, 128), x, "bf16")
    assert_close(ybig[:, :128].cpu().numpy(), yref, s, what="strided")
    assert torch.all(ybig[:, 128:] == 5.0)


def test_corrupt_tile_index_is_skipped():
    """tidx entries naming slots outside the streams are skipped by the
    kernels' own bounds checks (no access outside the buffers)."""
    torch = _torch()
    note("corrupt tidx")
    w, tmap = random_case(17, 128, 256, 64, 128, "bf16")
    P = pack_gpu(w, tmap, 64, 128, "bf16", "idx2")
    tid = P.tidx.cpu().numpy().copy()
    bad = tid.copy()
    bad[0] = 1 << 30          # dense slot far out of range
    bad[-1] = -(1 << 30)      # sparse slot far out of range
    P.tidx.copy_(torch.from_numpy(bad))
    x = wl.float32_to_bits(np.random.default_rng(3).standard_normal((2, 256)).astype(np.float32), "bf16")
    y = hb.gemv(P, upload(x, "bf16")).cpu().numpy()
    y2 = hb.gemm_mfma(P, upload(x, "bf16")).cpu().numpy()
    # the rows of the remaining tiles are still right
    keep = tmap.copy()
    wp = oracle.prune(w, tmap, 64, 128)
    wp[0:64, 0:128] = 0
    wp[64:128, 128:256] = 0
    yref, s = oracle.ref_matmul(wp, x, "bf16")
    assert_close(y, yref, s, what="gemv corrupt")
    assert_close(y2, yref, s, what="gemm corrupt")
    del keep


def test_gemm_millions_of_tokens_one_row_block():
    """4.3 million tokens on a 64 x 64 matrix: the register-fed shapes would
    need more token blocks than their grid allows (65535), so the launcher
    keeps the LDS-fed kernel (1-D grid); 2000 sampled tokens against the
    oracle."""
    torch = _torch()
    note("gemm 4.3M tokens, 64x64")
    n = k = b1 = b2 = 64
    m = 4_300_000
    w, tmap = random_case(4300, n, k, b1, b2, "bf16")
    rng = np.random.default_rng(4300)
    x = wl.float32_to_bits(rng.standard_normal((m, k), dtype=np.float32), "bf16")
    P = pack_gpu(w, tmap, b1, b2, "bf16", "idx2")
    y = hb.gemm(P, upload(x, "bf16"))
    torch.cuda.synchronize()
    pick = np.sort(rng.choice(m, size=2000, replace=False))
    pick[-1] = m - 1
    ys = y[torch.from_numpy(pick).to(dev())].cpu().numpy()
    yref, s = oracle.ref_matmul(oracle.prune(w, tmap, b1, b2), x[pick], "bf16")
    assert_close(ys, yref, s, what="4.3M tokens")


def test_corrupt_tile_index_and_16bit_out_lds_shape():
    """The LDS-fed kernel (8192 rows at 1024 tokens: the 128-token shape on
    a 256-CU device) skips tidx entries naming slots outside the streams,
    and rounds a bf16 y once; checked on tile rows that include the two
    corrupted tiles."""
    torch = _torch()
    note("corrupt tidx and bf16 y, lds shape")
    b1, b2, n, k, m = 64, 128, 8192, 256, 1024
    w, tmap = random_case(8191, n, k, b1, b2, "bf16")
    P = pack_gpu(w, tmap, b1, b2, "bf16", "idx2")
    bad = P.tidx.cpu().numpy().copy()
    tk = k // b2
    t0, t1 = 0, 5 * tk + 1            # tile (0, 0) and tile (5, 1)
    bad[t0] = 1 << 30                 # a dense slot far out of range
    bad[t1] = -(1 << 30)              # a sparse slot far out of range
    P.tidx.copy_(torch.from_numpy(bad))
    x = wl.float32_to_bits(np.random.default_rng(8191).standard_normal((m, k)).astype(np.float32), "bf16")
    xt = upload(x, "bf16")
    y = hb.gemm(P, xt).cpu().numpy()
    y16 = oracle.widen(hb.tensor_to_bits(hb.gemm(P, xt, out_dtype=torch.bfloat16)), "bf16")
    tile_rows = np.array([0, 5, 77])
    rows = np.concatenate([np.arange(tr * b1, (tr + 1) * b1) for tr in tile_rows])
    wp = oracle.prune(w[rows], tmap[tile_rows], b1, b2)
    wp[0:b1, 0:b2] = 0                # tile (0, 0) skipped
    wp[b1:2 * b1, b2:2 * b2] = 0      # tile (5, 1) skipped
    yref, s = oracle.ref_matmul(wp, x, "bf16")
    assert_close(y[:, rows], yref, s, what="lds corrupt tidx")
    assert_close(y16[:, rows], yref, s, extra=np.abs(yref) * 2.0 ** -8 + 2.0 ** -133, what="lds bf16 y")


def test_deterministic():
    torch = _torch()
    note("determinism")
    mat, w, tmap = workload_matrix(2, 0)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    x = upload(mat.activation_bits(4), "bf16")
    a = hb.gemv(P, x).cpu().numpy()
    b = hb.gemv(P, x).cpu().numpy()
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_all_dense_matches_torch_matmul():
    """Independent check of the dense path: hipBLAS via torch.matmul."""
    torch = _torch()
    note("dense vs torch.matmul")
    mat, w, _ = workload_matrix(2, 0)
    tmap = np.zeros((mat.tiles_n, mat.tiles_k), np.uint8)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    x = upload(mat.activation_bits(2), "bf16")
    y = hb.gemv(P, x)
    wt = upload(w, "bf16").float()
    yt = x.float() @ wt.t()
    s = x.float().abs() @ wt.abs().t()
    assert torch.all((y - yt).abs() <= 4e-3 * s + 1e-6)


def test_stream_read_reads_every_byte_once():
    """The streaming-read reference visits every 4-byte word exactly once:
    the XOR of its per-thread sinks equals the XOR of the buffer."""
    torch = _torch()
    note("stream read")
    rng = np.random.default_rng(21)
    words = rng.integers(0, 1 << 32, size=(3 << 18) + 100, dtype=np.uint32)   # not a multiple of 4 KiB
    buf = torch.from_numpy(words.view(np.int32)).to(dev())
    for grid in (1, 7, 512):
        sink = torch.zeros(grid * 256, dtype=torch.int32, device=dev())
        hb.stream_read(buf, words.nbytes, sink, grid)
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(words)


# ------------------------------------------- slot order and save / load ----

def _permuted(P, seed):
    """The same packed weight with its dense slots and its sparse slots in a
    random order: each slot's bytes move to the new position and tidx names
    the new slot."""
    torch = _torch()
    L = P.layout
    rng = np.random.default_rng(seed)
    pd = rng.permutation(L.n_dense)
    ps = rng.permutation(L.n_sparse)
    tile = L.b1 * L.b2
    def move(buf, count, per, perm):
        if count == 0:
            return buf.clone()
        src = buf.view(count, per)
        out = torch.empty_like(src)
        out[torch.from_numpy(perm).to(buf.device)] = src
        return out.view(-1)
    dense = move(P.dense, L.n_dense, tile * 2, pd)
    val = move(P.val, L.n_sparse, tile, ps)
    meta = move(P.meta, L.n_sparse, tile // 8, ps)
    t = P.tidx.cpu().numpy()
    t2 = np.where(t >= 0, pd[np.maximum(t, 0)] if L.n_dense else t,
                  ~(ps[np.maximum(~t, 0)] if L.n_sparse else ~t)).astype(np.int32)
    return hb.PackedWeight(L, dense, val, meta, torch.from_numpy(t2).to(P.device), P.dtype, P.meta_kind)


@pytest.mark.parametrize("meta", ["idx2", "mask8"])
def test_slot_order_does_not_change_results(meta):
    """Slots are names only: with the dense and sparse slots permuted (bytes
    moved, tidx renamed) unpack and every product kernel -- the decode
    kernel, the register-fed and the LDS-fed matrix-core kernels -- give
    bitwise the same results."""
    torch = _torch()
    note(f"slot order {meta}")
    n, k, b1, b2 = 8192, 512, 128, 128
    w, tmap = random_case(91, n, k, b1, b2, "bf16", frac=0.6)
    P = pack_gpu(w, tmap, b1, b2, "bf16", meta)
    Q = _permuted(P, 5)
    assert torch.equal(hb.unpack(P), hb.unpack(Q))
    for m in (1, 5, 16, 40, 300, 1024):
        x = upload(wl.float32_to_bits(np.random.default_rng(m).standard_normal((m, k)).astype(np.float32),
                                      "bf16"), "bf16")
        assert torch.equal(hb.gemm(P, x), hb.gemm(Q, x)), m
    torch.cuda.synchronize()


def test_save_load_gpu_round_trip(tmp_path):
    """A packed weight saved from the GPU and loaded back gives bitwise the
    same decode and prefill products."""
    torch = _torch()
    note("save / load round trip")
    mat, w, tmap = workload_matrix(1, 0)
    P = pack_gpu(w, tmap, mat.b1, mat.b2, mat.dtype, "idx2")
    path = tmp_path / "w.hyb"
    hb.save(P, path)
    Q = hb.load(path, dev())
    for m in (1, 64):
        x = upload(mat.activation_bits(m), mat.dtype)
        assert torch.equal(hb.gemm(P, x), hb.gemm(Q, x)), m
