"""The allocation-free refine entry point (prism_refine_attend_static, scratch in the library's
static device array) against the workspace entry point (prism_refine_attend) on the same inputs,
through the C ABI: two calls in a row on one GPU, the second with a smaller input, each equal to
the workspace call bit for bit (same kernels and launch shapes), and the first also against the
oracle's tie band and tolerances."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from tests.parity import check_refine_batch, dev, host
from token_level_sparse_prism_amd import binding as PB

pytestmark = pytest.mark.gpu


def _inputs(seed, Bn, Hq, Hkv, D, T, lens):
    rng = np.random.default_rng(seed)
    f = lambda *s: PB_round(rng.standard_normal(s).astype(np.float32))
    q, K, V = f(Bn, Hq, D), f(Bn, Hkv, T, D), f(Bn, Hkv, T, D)
    lens = np.asarray(lens, np.int32)
    for b in range(Bn):
        K[b, :, lens[b]:] = 0.0
        V[b, :, lens[b]:] = 0.0
    q0 = PB_round(rng.standard_normal((Bn, Hq, D)).astype(np.float32))
    return q, K, V, lens, q0


def PB_round(x):
    from token_level_sparse_prism_amd import workload as W
    return W.bf16_round(x)


@pytest.mark.parametrize("first,second", [
    # (B, Hq, Hkv, D, T, kp, kappa, lens): a larger call, then a smaller one on the same scratch
    ((2, 32, 8, 128, 20000, 4096, 1024, [20000, 13000]), (1, 8, 2, 64, 6000, 1500, 300, [5000])),
    ((1, 32, 8, 128, 65536, 8192, 2048, [65536]), (1, 4, 1, 128, 3000, 1000, 1000, [3000])),
])
def test_static_matches_workspace_entry(first, second):
    lib = PB.load()
    for n, (Bn, Hq, Hkv, D, T, kp, kappa, lens) in enumerate((first, second)):
        q, K, V, lens, q0 = _inputs(1000 * n + T, Bn, Hq, Hkv, D, T, lens)
        Kq, sc = oracle.quantize_rows(K)
        pool = oracle.propose(q0, Kq, sc, kp, seq_lens=lens)
        qd, Kd, Vd = dev(q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
        pd, ld = torch.from_numpy(pool).cuda(), torch.from_numpy(lens).cuda()
        ref = PB.refine_attend(qd, Kd, Vd, pd, kappa, seq_lens=ld)
        out = torch.full_like(ref[0], 7.0)
        idx = torch.full_like(ref[1], 7)
        lse = torch.full_like(ref[2], 7.0)
        torch.cuda.synchronize()
        shape = PB.make_shape(qd, Kd, ld)
        rc = lib.prism_refine_attend_static(PB._ptr(qd), PB._ptr(Kd), PB._ptr(Vd), PB.PRISM_BF16, ctypes.byref(shape),
                                            PB._ptr(pd), kp, kappa, PB.AGG_SUM, 0.0, PB._ptr(out), PB._ptr(idx),
                                            PB._ptr(lse), None)
        assert rc == 0, PB.STATUS.get(rc, rc)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[1]), f"call {n}: idx"
        assert torch.equal(out, ref[0]), f"call {n}: out"
        assert torch.equal(lse, ref[2]), f"call {n}: lse"
        check_refine_batch(idx.cpu().numpy(), host(out), lse.cpu().numpy(), q, K, V, lens, pool, kappa, PB.AGG_SUM,
                           "bf16")


def test_static_rejects_what_does_not_fit():
    """A refine layout above the 32 MiB scratch is rejected before any device work."""
    lib = PB.load()
    f = ctypes.c_void_p
    big = PB.Shape(1, 64, 64, 256, 1 << 20, None)   # 64 units, kp = 2^20: far above 32 MiB
    rc = lib.prism_refine_attend_static(f(256), f(256), f(256), PB.PRISM_BF16, ctypes.byref(big), f(256), 1 << 20,
                                        2048, 0, 0.0, f(256), f(256), None, None)
    assert rc == 3
