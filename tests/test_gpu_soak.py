"""Soak of the attention's cross-workgroup hand-off (split partials written with device-coherent
stores, an arrival counter, the last workgroup's merge): a whole step captured in a HIP graph and
replayed 2000 times per shape, every replay's pools, index sets, outputs and lse compared bit for bit
with the eager step on the device, checked every 200 replays and at the end (the first bad batch
fails the test).  Every shape takes the rank-split attention, the one with the hand-off (kappa above
what the head-dimension split takes, or more units than its grid fits): one unit and five units at
kappa = 4096 (their attention workgroups fall on several XCDs, so partials cross XCDs, and 32 slices
per unit take the two-level merge) and 64 units at kappa = 1024 (each unit's workgroups on one XCD)."""
import pytest
import torch

from token_level_sparse_prism_amd import binding as PB
from token_level_sparse_prism_amd import workload as W
from token_level_sparse_prism_amd.step import LayerInputs, PrismStep

pytestmark = pytest.mark.gpu

SHAPES = [
    # name, config overrides
    ("1 unit", dict(B=1, Hq=8, Hkv=1, T=65536, kp=8192, kappa=4096, n_refined=3)),
    ("5 units", dict(B=1, Hq=20, Hkv=5, T=32768, kp=8192, kappa=4096, n_refined=3)),
    ("64 units", dict(B=8, Hq=32, Hkv=8, T=20000, kp=4096, kappa=1024, n_refined=3, seq_lens=None)),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,ov", SHAPES, ids=[s[0].replace(" ", "") for s in SHAPES])
def test_graph_replay_soak(name, ov):
    c = W.CONFIGS["cfg2"].with_(**ov)
    # the launcher takes the head-dimension split (no hand-off) for kappa <= 2048 when the unit count
    # times the D / 8 sixteen-byte bf16 pieces fits the CUs; keep every shape off it
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert c.kappa > 2048 or c.B * c.Hkv * (c.D // 8) > cus, "shape would not exercise the hand-off"
    w = W.generate(c)
    dev = lambda x: torch.from_numpy(x).to(device="cuda", dtype=torch.bfloat16)
    ld = torch.from_numpy(w.seq_lens).cuda()
    Kq, sc = PB.quantize_keys(dev(w.K[0]), seq_lens=ld)
    step = PrismStep(dev(w.q[0]), Kq, sc, [LayerInputs(dev(w.q[l]), dev(w.K[l]), dev(w.V[l])) for l in range(1, w.layers)],
                     c.kp, c.kappa, seq_lens=ld)
    step()
    torch.cuda.synchronize()
    outs = [step.pool] + list(step.idx) + list(step.out) + list(step.lse)
    ref = [t.clone() for t in outs]
    graph = step.capture()
    bad = torch.zeros((), dtype=torch.bool, device="cuda")
    for i in range(2000):
        graph.replay()
        for a, b in zip(outs, ref):
            bad |= (a != b).any()
        if (i + 1) % 200 == 0:
            assert not bool(bad.item()), f"{name}: a replay in the batch ending at {i + 1} differs from the eager step"
