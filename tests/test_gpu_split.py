"""GPU parity of the split-K launches (k_gemm_split, the register-fed
shapes; k_gemm_lds_split, the LDS-fed 64- and 128-token shapes; and
k_gemm_lds_parts, the 192- and 256-token LDS tiles with K cut into equal
parts; each followed by
the kernel that adds its partial tiles): every split shape the launcher
uses, in every dtype, metadata kind and tile size, with ragged row and token
blocks, the low-rank epilogue, corrupt tile indices, 16-bit outputs, the
caller-held workspace of hyb_gemm_ws, and replays of a captured graph.
Every output against the oracle (same acceptance rule as test_gpu_parity)."""
import numpy as np
import pytest

import oracle
from matmul_pack_b1_amd import binding as hb
from matmul_pack_b1_amd import workloads as wl
from test_gpu_parity import (_torch, assert_close, dev, expect_route, note, oracle_full, oracle_full_lowrank,
                             pack_gpu, random_case, upload)

pytestmark = pytest.mark.gpu

# (n, k, b1, b2, m, dtype, meta) -> split shape (token blocks, wavefronts,
# row groups) on a 256-CU device; row groups 4 is the LDS-fed shape.  2112
# rows leave the last 128-row block half outside the matrix, 8256, 8320,
# 16448, 32832, 2880, 3008, 3200, 8256, 10816, 11136, 2496, 3392, 3136,
# 2112, 2432, 3904, 4032 and 1984 the last 256-row block; 100, 90, 70, 60,
# 49, 120, 150, 180, 200, 300, 400, 450 and 500 tokens leave a ragged token
# block (2 to 4 token blocks at 300-500).
CASES = [
    ((256, 4096, 128, 128, 33, "bf16", "idx2"), (1, 8, 1)),
    ((192, 8192, 64, 128, 17, "f16", "mask8"), (1, 8, 1)),
    ((1024, 16384, 64, 256, 20, "f16", "mask4"), (2, 8, 1)),
    ((4096, 16384, 64, 128, 20, "bf16", "mask4"), (2, 4, 2)),
    ((2048, 8192, 256, 64, 65, "bf16", "mask8"), (3, 4, 2)),
    ((2112, 16384, 64, 128, 70, "bf16", "mask4"), (3, 4, 2)),
    ((1024, 16384, 64, 64, 48, "bf16", "mask4"), (3, 4, 2)),
    ((2112, 16384, 64, 128, 90, "f16", "mask8"), (3, 4, 2)),
    ((1088, 8192, 64, 128, 100, "f16", "idx2"), (4, 8, 1)),
    ((2048, 16384, 128, 128, 100, "f16", "idx2"), (4, 4, 2)),
    ((2112, 16384, 64, 128, 100, "bf16", "idx2"), (4, 4, 2)),
    ((8256, 5120, 64, 64, 100, "bf16", "idx2"), (4, 8, 4)),
    ((8320, 5120, 128, 128, 120, "f16", "mask8"), (4, 8, 4)),
    ((8448, 6144, 256, 64, 100, "bf16", "mask8"), (8, 8, 4)),
    ((16448, 4096, 64, 256, 64, "f16", "idx2"), (4, 8, 4)),
    ((16512, 4096, 128, 128, 49, "bf16", "mask4"), (4, 8, 4)),
    ((32832, 2048, 64, 128, 100, "bf16", "idx2"), (4, 8, 4)),
    ((7616, 8192, 64, 64, 128, "f16", "mask4"), (8, 8, 4)),
    ((15296, 8192, 64, 64, 60, "f16", "mask8"), (4, 8, 4)),
    ((2880, 16384, 64, 64, 100, "bf16", "idx2"), (8, 8, 4)),
    ((3008, 16384, 64, 128, 120, "f16", "mask4"), (8, 8, 4)),
    ((3200, 16384, 128, 128, 128, "bf16", "mask8"), (8, 8, 4)),
    ((3840, 12288, 256, 64, 128, "bf16", "idx2"), (8, 8, 4)),
    ((8256, 8192, 64, 256, 300, "f16", "idx2"), (8, 8, 4)),
    ((10816, 5120, 64, 64, 300, "bf16", "mask4"), (8, 8, 4)),
    ((11136, 8192, 64, 128, 400, "bf16", "idx2"), (8, 8, 4)),
    ((2496, 12288, 64, 64, 450, "f16", "mask8"), (16, 8, 4)),
    ((3392, 16384, 64, 64, 200, "bf16", "idx2"), (16, 8, 4)),
    ((3136, 16384, 64, 128, 256, "f16", "mask4"), (16, 8, 4)),
    ((2112, 16384, 64, 256, 500, "bf16", "mask8"), (16, 8, 4)),
    ((2432, 12288, 128, 64, 400, "f16", "idx2"), (16, 8, 4)),
    ((3072, 16384, 256, 256, 400, "bf16", "mask4"), (16, 8, 4)),
    ((3904, 16384, 64, 64, 150, "bf16", "idx2"), (12, 8, 4)),
    ((4032, 16384, 64, 128, 180, "f16", "mask8"), (12, 8, 4)),
    ((3008, 16384, 64, 64, 300, "bf16", "mask4"), (12, 8, 4)),
    ((1984, 12288, 64, 128, 500, "f16", "idx2"), (12, 8, 4)),
    ((4096, 16384, 256, 128, 300, "bf16", "mask8"), (12, 8, 4)),
]

# One product per split kernel for the checks below: (n, k, b, m) -> shape.
KERNELS = [((2048, 16384, 128, 100), (4, 4, 2)), ((8320, 5120, 128, 100), (4, 8, 4)),
           ((3200, 16384, 128, 120), (8, 8, 4)), ((3136, 16384, 64, 256), (16, 8, 4))]


def _case(n, k, b1, b2, m, dtype, meta):
    w, tmap = random_case(n + k + m, n, k, b1, b2, dtype, frac=0.6)
    x = wl.float32_to_bits(np.random.default_rng(n + m).standard_normal((m, k)).astype(np.float32), dtype)
    return w, tmap, x


@pytest.mark.parametrize("case,shape", CASES)
def test_split_shapes_every_output(case, shape):
    """hyb_gemm (torch workspace), hyb_gemm_mfma (library-held workspace) and
    hyb_gemm_ws with an explicit workspace give the same bits (same launch);
    hyb_gemm_ws without a workspace runs the same shape unsplit.  All four
    against the oracle on every output; a second call repeats the bits."""
    torch = _torch()
    n, k, b1, b2, m, dtype, meta = case
    note(f"split {case}")
    w, tmap, x = _case(*case)
    P = pack_gpu(w, tmap, b1, b2, dtype, meta)
    expect_route(P, m, "split", *shape)
    need = hb.workspace_bytes(P, m)
    assert 0 < need <= 64 << 20
    xt = upload(x, dtype)
    y = hb.gemm(P, xt)
    y_again = hb.gemm(P, xt)
    y_held = hb.gemm_mfma(P, xt)
    ws = torch.empty(need + 256, dtype=torch.uint8, device=dev())
    y_ws = hb.gemm(P, xt, workspace=ws)
    y_plain = hb.gemm(P, xt, workspace=torch.empty(0, dtype=torch.uint8, device=dev()))
    torch.cuda.synchronize()
    for other in (y_again, y_held, y_ws):
        assert torch.equal(y.view(torch.int32), other.view(torch.int32))
    yref, s = oracle_full(w, tmap, b1, b2, x, dtype, meta)
    assert_close(y.cpu().numpy(), yref, s, what=f"split {case}")
    assert_close(y_plain.cpu().numpy(), yref, s, what=f"unsplit {case}")


@pytest.mark.parametrize("case,shape", [((2112, 16384, 64, 128, 100), (4, 4, 2)), ((8256, 5120, 64, 64, 100), (4, 8, 4)),
                                        ((8256, 8192, 64, 128, 300), (8, 8, 4)),
                                        ((3904, 16384, 64, 128, 150), (12, 8, 4)),
                                        ((3392, 16384, 64, 128, 200), (16, 8, 4))])
def test_split_lowrank_and_bf16_out(case, shape):
    """The low-rank term is added by the piece that starts at K step 0, and
    the split tiles' sums are rounded once to a bf16 y."""
    torch = _torch()
    n, k, b1, b2, m = case
    rank = 64
    note(f"split lowrank + bf16 y {case}")
    w, tmap, x = _case(n, k, b1, b2, m, "bf16", "idx2")
    rng = np.random.default_rng(99)
    t = (rng.standard_normal((m, rank)) * 4).astype(np.float32)
    u = wl.float32_to_bits(rng.standard_normal((n, rank)).astype(np.float32) * 0.05, "bf16")
    P = pack_gpu(w, tmap, b1, b2, "bf16", "idx2")
    expect_route(P, m, "split", *shape)
    xt, tt = upload(x, "bf16"), torch.from_numpy(t).to(dev())
    y = hb.gemm_lowrank(P, xt, tt, upload(u, "bf16"))
    y16 = oracle.widen(hb.tensor_to_bits(hb.gemm(P, xt, out_dtype=torch.bfloat16)), "bf16")
    torch.cuda.synchronize()
    yref, s = oracle_full_lowrank(w, tmap, b1, b2, x, t, u, "bf16")
    assert_close(y.cpu().numpy(), yref, s, what="split lowrank")
    y0ref, s0 = oracle_full(w, tmap, b1, b2, x, "bf16")
    assert_close(y16, y0ref, s0, extra=np.abs(y0ref) * 2.0 ** -8 + 2.0 ** -133, what="split bf16 y")


@pytest.mark.parametrize("case,shape", KERNELS)
def test_split_skips_corrupt_tile_index(case, shape):
    """tidx entries naming slots outside the streams are skipped inside the
    split pieces too (the kernels' own bounds checks)."""
    torch = _torch()
    n, k, b, m = case
    b1 = b2 = b
    note(f"split corrupt tidx {case}")
    w, tmap, x = _case(n, k, b1, b2, m, "f16", "idx2")
    P = pack_gpu(w, tmap, b1, b2, "f16", "idx2")
    expect_route(P, m, "split", *shape)
    tk = k // b2
    bad = P.tidx.cpu().numpy().copy()
    c0 = tk // 3
    t0, t1 = 3 * tk + c0, 9 * tk + tk - 1      # tile (3, tk / 3) and tile (9, last)
    bad[t0] = 1 << 30
    bad[t1] = -(1 << 30)
    P.tidx.copy_(torch.from_numpy(bad))
    y = hb.gemm(P, upload(x, "f16")).cpu().numpy()
    wp = oracle.prune(w, tmap, b1, b2)
    wp[3 * b1:4 * b1, c0 * b2:(c0 + 1) * b2] = 0
    wp[9 * b1:10 * b1, (tk - 1) * b2:tk * b2] = 0
    yref, s = oracle.ref_matmul(wp, x, "f16")
    assert_close(y, yref, s, what="split corrupt tidx")


@pytest.mark.parametrize("case,shape", KERNELS)
def test_split_in_a_captured_graph(case, shape):
    """A split product captured into a graph: each of three replays, with
    eager work and synchronisations between them, gives the eager bits."""
    torch = _torch()
    n, k, b, m = case
    b1 = b2 = b
    note(f"split graph replays {case}")
    w, tmap, x = _case(n, k, b1, b2, m, "bf16", "idx2")
    P = pack_gpu(w, tmap, b1, b2, "bf16", "idx2")
    expect_route(P, m, "split", *shape)
    xt = upload(x, "bf16")
    eager = hb.gemm(P, xt)
    y = torch.empty_like(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        g.capture_begin()
        hb.gemm(P, xt, out=y)
        g.capture_end()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    for i in range(3):
        y.fill_(float("nan"))
        hb.gemm(P, xt[: m // 2])            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), eager.view(torch.int32)), f"replay {i}"
    del g


def test_split_workspace_checks():
    """hyb_gemm_ws rejects a workspace below the need, before any launch."""
    torch = _torch()
    n, k, b1, b2, m = 2048, 16384, 128, 128, 100
    w, tmap, x = _case(n, k, b1, b2, m, "bf16", "idx2")
    P = pack_gpu(w, tmap, b1, b2, "bf16", "idx2")
    need = hb.workspace_bytes(P, m)
    small = torch.empty(need - 16, dtype=torch.uint8, device=dev())
    with pytest.raises(hb.HybError) as e:
        hb.gemm(P, upload(x, "bf16"), workspace=small)
    assert e.value.status == 1


def test_split_two_streams_held_workspaces():
    """hyb_gemm_mfma keeps one workspace per (device, stream): split products
    enqueued on two streams at once, each on its own inputs, give the bits of
    the same products run one after the other."""
    torch = _torch()
    n, k, b1, b2 = 2048, 16384, 128, 128
    note("split on two streams")
    cases = []
    for m, seed in ((100, 1), (48, 2)):
        w, tmap = random_case(seed, n, k, b1, b2, "bf16", frac=0.6)
        x = wl.float32_to_bits(np.random.default_rng(seed).standard_normal((m, k)).astype(np.float32), "bf16")
        P = pack_gpu(w, tmap, b1, b2, "bf16", "idx2")
        assert hb.gemm_shape(P.layout, m)["kernel"] == "split"
        cases.append((P, upload(x, "bf16")))
    serial = [hb.gemm_mfma(P, x) for P, x in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(y) for y in serial]
    for rep in range(3):
        for s_ in streams:
            s_.wait_stream(torch.cuda.current_stream())
        for (P, x), s_, out in zip(cases, streams, outs):
            with torch.cuda.stream(s_):
                for _ in range(4):
                    hb.gemm_mfma(P, x, out=out)
        torch.cuda.synchronize()
        for y, out in zip(serial, outs):
            assert torch.equal(y.view(torch.int32), out.view(torch.int32)), f"repeat {rep}"


# Whole rounds of plain 256-token tiles, then the last 256-row blocks with K
# cut into parts (k_gemm_lds over the first blocks, k_gemm_lds_parts and its
# sum over the rest): (n, k, b1, b2, m, dtype, meta) -> workgroups of the
# parts launch on a 256-CU device.  16640 rows are 65 blocks of 256: at 4
# token blocks 64 blocks fill one round, and the 65th block's 4 tiles run in
# 4 K parts; 16704 rows add a 66th block a quarter full; 900 and 1000 tokens
# leave a ragged token block.
TAIL_CASES = [
    ((16640, 4096, 128, 128, 1000, "bf16", "idx2"), 16),
    ((16640, 4096, 64, 64, 1024, "f16", "mask4"), 16),
    ((16640, 4096, 256, 256, 900, "bf16", "mask8"), 16),
    ((16704, 4096, 64, 128, 1000, "bf16", "idx2"), 32),
]


@pytest.mark.parametrize("case,tail_wgs", TAIL_CASES)
def test_lds_tail_every_output(case, tail_wgs):
    """The route and its workspace (one 256-row x 256-token partial tile per
    parts workgroup); hyb_gemm, hyb_gemm_noalloc and a second call give the
    same bits; hyb_gemm_ws without a workspace runs every tile plain.  Both
    against the oracle on every output, so the rows on either side of the
    boundary between the two launches are covered."""
    torch = _torch()
    n, k, b1, b2, m, dtype, meta = case
    note(f"lds tail {case}")
    w, tmap, x = _case(*case)
    P = pack_gpu(w, tmap, b1, b2, dtype, meta)
    expect_route(P, m, "split", 16, 8, 4)
    assert hb.workspace_bytes(P, m) == tail_wgs * 256 * 256 * 4
    xt = upload(x, dtype)
    y = hb.gemm(P, xt)
    y_again = hb.gemm(P, xt)
    y_static = hb.gemm_noalloc(P, xt)
    y_plain = hb.gemm(P, xt, workspace=torch.empty(0, dtype=torch.uint8, device=dev()))
    torch.cuda.synchronize()
    for other in (y_again, y_static):
        assert torch.equal(y.view(torch.int32), other.view(torch.int32))
    yref, s = oracle_full(w, tmap, b1, b2, x, dtype, meta)
    assert_close(y.cpu().numpy(), yref, s, what=f"lds tail {case}")
    assert_close(y_plain.cpu().numpy(), yref, s, what=f"plain {case}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_lds_tail_lowrank_and_16bit_out(dtype):
    """On the same route the low-rank rows of the parts launch are those of
    its row blocks (U moves with the view), T U^T is added once, and a bf16
    y is rounded once; the caller-workspace and library-workspace entry
    points give the same bits, also from a captured graph."""
    torch = _torch()
    n, k, b1, b2, m = 16704, 4096, 64, 128, 1000
    rank = 32
    note(f"lds tail lowrank + 16-bit y {dtype}")
    w, tmap, x = _case(n, k, b1, b2, m, dtype, "idx2")
    rng = np.random.default_rng(1000)
    t = (rng.standard_normal((m, rank)) * 4).astype(np.float32)
    u = wl.float32_to_bits(rng.standard_normal((n, rank)).astype(np.float32) * 0.05, dtype)
    P = pack_gpu(w, tmap, b1, b2, dtype, "idx2")
    expect_route(P, m, "split", 16, 8, 4)
    xt, tt = upload(x, dtype), torch.from_numpy(t).to(dev())
    ut = upload(u, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    y = hb.gemm_lowrank(P, xt, tt, ut)
    y_held = hb.gemm_lowrank_held(P, xt, tt, ut)
    y16 = oracle.widen(hb.tensor_to_bits(hb.gemm(P, xt, out_dtype=tdt)), dtype)
    # captured with the workspace from torch's allocator, the graph runs the
    # same split launches: three replays give the eager bits
    yg = torch.empty_like(y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        g.capture_begin()
        hb.gemm_lowrank(P, xt, tt, ut, out=yg)
        g.capture_end()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y_held.view(torch.int32))
    for i in range(3):
        yg.fill_(float("nan"))
        hb.gemm(P, xt[: m // 2])            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg.view(torch.int32), y.view(torch.int32)), f"replay {i}"
    del g
    yref, s = oracle_full_lowrank(w, tmap, b1, b2, x, t, u, dtype)
    assert_close(y.cpu().numpy(), yref, s, what="lds tail lowrank")
    y0ref, s0 = oracle_full(w, tmap, b1, b2, x, dtype)
    # half an output ulp of rounding on top of the bound (bf16: 2^-8 relative,
    # fp16: 2^-11 relative and 2^-25 absolute below its normal range)
    ulp = (np.abs(y0ref) * 2.0 ** -8 + 2.0 ** -133) if dtype == "bf16" else (np.abs(y0ref) * 2.0 ** -11 + 2.0 ** -25)
    assert_close(y16, y0ref, s0, extra=ulp, what=f"lds tail {dtype} y")
