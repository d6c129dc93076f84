"""hyb_gemm_noalloc (the entry point for callers that cannot allocate)
against hyb_gemm on the same inputs: two calls in a row on split routes, the
second with a smaller input, plus an unsplit and a decode-kernel call; the
same bits as hyb_gemm (same kernels and schedule) and every output within
the oracle's bound."""
import numpy as np
import pytest

from matmul_pack_b1_amd import binding as hb
from matmul_pack_b1_amd import workloads as wl
from test_gpu_parity import _torch, assert_close, expect_route, note, oracle_full, pack_gpu, random_case, upload

pytestmark = pytest.mark.gpu


def _product(n, k, b1, b2, m, dtype, meta, seed):
    w, tmap = random_case(seed, n, k, b1, b2, dtype, frac=0.6)
    x = wl.float32_to_bits(np.random.default_rng(seed + 1).standard_normal((m, k)).astype(np.float32), dtype)
    return w, tmap, x


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_gemm(order):
    torch = _torch()
    cases = [
        ((11136, 8192, 64, 128, 400, "bf16", "idx2"), ("split", 8, 8, 4)),    # all 64 MiB of scratch in use
        ((3136, 16384, 64, 128, 256, "f16", "mask4"), ("split", 16, 8, 4)),   # K cut in parts: 52 MiB
        ((8256, 5120, 64, 64, 100, "bf16", "idx2"), ("split", 4, 8, 4)),      # 32 MiB
        ((2048, 16384, 128, 128, 100, "bf16", "idx2"), ("split", 4, 4, 2)),   # 16 MiB
        ((256, 4096, 128, 128, 33, "f16", "mask4"), ("split", 1, 8, 1)),      # smaller: reuses the array
        ((1024, 4096, 128, 128, 384, "bf16", "idx2"), ("register", 2, 8, 1)),
        ((1024, 4096, 128, 128, 4, "bf16", "mask8"), ("decode", None, None, None)),
    ]
    for (n, k, b1, b2, m, dtype, meta), route in cases:
        note(f"noalloc {n}x{k} m={m} {dtype} {meta}")
        w, tmap, x = _product(n, k, b1, b2, m, dtype, meta, n + m)
        P = pack_gpu(w, tmap, b1, b2, dtype, meta)
        expect_route(P, m, *route)
        xt = upload(x, dtype)
        ref = hb.gemm(P, xt)
        y = hb.gemm_noalloc(P, xt)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), (n, k, m)
        yref, s = oracle_full(w, tmap, b1, b2, x, dtype, meta)
        assert_close(y.cpu().numpy(), yref, s, what=f"noalloc {n}x{k} m={m}")
