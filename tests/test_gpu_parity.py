"""GPU parity: the HIP path through the C ABI against the CPU oracle, on seeded inputs.

Sizes span several 1024-token chunks with a ragged tail; shapes cover D in {64, 128, 256},
G in {1, 3 (padded to 4), 4, 8, 16}, fp32 and bf16, SUM and MAX aggregation, ragged and empty
sequences, kp above T_b, heavy score ties and the q = 0 degenerate case.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from tests.parity import (assert_pool_equal, check_dense_batch, check_refine_batch, dev, f32_bits, host,
                          unpack_int2)
from token_level_sparse_prism_amd import binding as PB
from token_level_sparse_prism_amd import workload as W

pytestmark = pytest.mark.gpu


def seed_of(*parts):
    return zlib.crc32(repr(parts).encode())


def rnd(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return W.bf16_round(x) if dtype == "bf16" else x


def make_inputs(seed, Bn, Hq, Hkv, D, T, dtype, lens=None, ties=False, zero_q=False, clustered=False, dup=0):
    rng = np.random.default_rng(seed)
    q = rnd(rng, (Bn, Hq, D), dtype)
    K = rnd(rng, (Bn, Hkv, T, D), dtype)
    V = rnd(rng, (Bn, Hkv, T, D), dtype)
    if ties:
        proto = rnd(rng, (7, D), dtype)
        K[:] = proto[rng.integers(0, 7, size=(Bn, Hkv, T))]
    if dup:
        # runs of `dup` equal rows: the threshold key is shared by up to `dup` pool slots, fewer
        # than the lean selection's short list holds, so its tie path ranks them
        K[:] = K[:, :, (np.arange(T) // dup) * dup]
    if clustered:
        # q.K = a + b / 256 per head with a in 1 + {0..15}/128 and b in 1 + {0..127}/128: 2048
        # distinct scores inside one octave's eighth (two for G = 3), exact in bf16 products and
        # fp32 sums, so both sides rank the same values; some tokens share a score
        K[:] = 0.0
        K[..., 0] = 1.0 + rng.integers(0, 16, size=(Bn, Hkv, T)) / 128.0
        K[..., 1] = 1.0 + rng.integers(0, 128, size=(Bn, Hkv, T)) / 128.0
        q[:] = 0.0
        q[..., 0] = 1.0
        q[..., 1] = 2.0 ** -8
    if zero_q:
        q[:] = 0.0
    lens = np.full(Bn, T, np.int32) if lens is None else np.asarray(lens, np.int32)
    for b in range(Bn):
        K[b, :, lens[b]:] = 0.0
        V[b, :, lens[b]:] = 0.0
    return q, K, V, lens


def gpu_quant(K, dtype, lens):
    Kd = dev(K, dtype)
    ld = torch.from_numpy(lens).cuda()
    Kq, sc = PB.quantize_keys(Kd, seq_lens=ld)
    torch.cuda.synchronize()
    return Kq, sc, ld


# ------------------------------------------------------------------------------------- quantize
@pytest.mark.parametrize("D,dtype,T,lens", [(128, "f32", 4096, None), (64, "bf16", 3000, [3000, 1777]),
                                            (256, "bf16", 2500, [0, 2500]), (128, "bf16", 5000, None)])
def test_quantize_keys_bitexact(D, dtype, T, lens):
    q, K, V, lens = make_inputs(D + T, 2 if lens else 1, 4, 2, D, T, dtype, lens)
    K[0, 0, 5] = 0.0  # an all-zero row
    Kq, sc, _ = gpu_quant(K, dtype, lens)
    Kq, sc = Kq.cpu().numpy(), sc.cpu().numpy()
    for b in range(K.shape[0]):
        n = lens[b]
        oq, os_ = oracle.quantize_rows(K[b, :, :n])
        assert np.array_equal(Kq[b, :, :n], oq)
        assert np.array_equal(f32_bits(sc[b, :, :n]), f32_bits(os_))


# ------------------------------------------------------------------------------------- propose
PROPOSE_CASES = [
    # D, G, Hkv, agg, dtype, T, kp, lens
    (128, 4, 2, PB.AGG_SUM, "bf16", 5000, 1024, None),
    (64, 8, 2, PB.AGG_SUM, "bf16", 9000, 4096, [9000, 3000]),
    (256, 1, 1, PB.AGG_SUM, "f32", 4096, 1024, None),
    (128, 3, 2, PB.AGG_MAX, "bf16", 6000, 512, None),
    (128, 4, 1, PB.AGG_MAX, "f32", 3000, 2999, None),
    (64, 16, 1, PB.AGG_SUM, "bf16", 2500, 100, None),
    (256, 8, 1, PB.AGG_MAX, "bf16", 2100, 2048, [2100, 1]),
    (128, 4, 2, PB.AGG_SUM, "bf16", 1000, 1500, None),   # kp > T: take everything
    (128, 4, 2, PB.AGG_SUM, "bf16", 3000, 700, [3000, 0]),  # an empty sequence
    (128, 1, 1, PB.AGG_SUM, "bf16", 1, 4, None),          # a single token
]


@pytest.mark.parametrize("case", PROPOSE_CASES, ids=lambda c: f"D{c[0]}G{c[1]}a{c[3]}{c[4]}T{c[5]}kp{c[6]}")
@pytest.mark.parametrize("variant", ["random", "ties", "zero_q"])
def test_propose_bitexact(case, variant):
    D, G, Hkv, agg, dtype, T, kp, lens = case
    Bn = len(lens) if lens else 1
    q, K, V, lens = make_inputs(seed_of(D, G, T, kp, variant), Bn, G * Hkv, Hkv, D, T, dtype, lens,
                                ties=variant == "ties", zero_q=variant == "zero_q")
    Kq, sc, ld = gpu_quant(K, dtype, lens)
    scores = torch.zeros((Bn, Hkv, T), dtype=torch.float32, device="cuda")
    pool = PB.propose(dev(q, dtype), Kq, sc, kp, agg, seq_lens=ld, scores=scores)
    torch.cuda.synchronize()
    oKq, osc = oracle.quantize_rows(K)
    opool, oscores = oracle.propose(q, oKq, osc, kp, seq_lens=lens, agg=agg, want_scores=True)
    gs = scores.cpu().numpy()
    for b in range(Bn):
        assert np.array_equal(f32_bits(gs[b, :, :lens[b]]), f32_bits(oscores[b, :, :lens[b]])), "scores differ"
    assert_pool_equal(pool.cpu().numpy(), opool)


SEL_WGS = 512  # the proposal selection's workgroup target (the launcher's PRISM_SEL_WGS)


def chunks_per_selection_wg(units, T):
    """M of the launcher: 1 while units x chunks <= SEL_WGS, else doubled (up to 8) until the
    grid of chunk groups is back at or below SEL_WGS * M."""
    nchunks = -(-T // 1024)
    m = 1
    while m < 8 and units * nchunks > SEL_WGS * m:
        m *= 2
    return m


# Grids of more than SEL_WGS chunk workgroups: the selection kernels take 2, 4 or 8 chunks per
# workgroup.  Every chunk count below is odd or no multiple of M, so the last group holds chunks
# past the key row; ragged and empty sequences put whole groups past T_b.
GROUPED_CASES = [
    # D, G, B, Hkv, T, kp, lens, expected M
    (128, 4, 2, 8, 33000, 1500, [33000, 17000], 2),                      # 16 units x 33 chunks
    (128, 4, 4, 16, 20000, 2000, [20000, 12345, 0, 7777], 4),            # 64 units x 20 chunks
    (64, 2, 4, 16, 41000, 4096, [41000, 40100, 1025, 41000], 8),         # 64 units x 41 chunks
    (64, 2, 8, 16, 33000, 3000, [33000, 1, 32768, 33000, 20000, 33000, 0, 9999], 8),  # 128 x 33
]


@pytest.mark.parametrize("case", GROUPED_CASES, ids=lambda c: f"U{c[2] * c[3]}T{c[4]}M{c[7]}")
@pytest.mark.parametrize("variant", ["random", "ties"])
def test_propose_grouped_chunks_bitexact(case, variant):
    D, G, Bn, Hkv, T, kp, lens, M = case
    assert chunks_per_selection_wg(Bn * Hkv, T) == M
    q, K, V, lens = make_inputs(seed_of(D, G, T, kp, variant), Bn, G * Hkv, Hkv, D, T, "bf16", lens,
                                ties=variant == "ties")
    Kq, sc, ld = gpu_quant(K, "bf16", lens)
    pool = PB.propose(dev(q, "bf16"), Kq, sc, kp, PB.AGG_SUM, seq_lens=ld)
    torch.cuda.synchronize()
    oKq, osc = oracle.quantize_rows(K)
    opool = oracle.propose(q, oKq, osc, kp, seq_lens=lens, agg=PB.AGG_SUM)
    assert_pool_equal(pool.cpu().numpy(), opool)


# ------------------------------------------------------------------------------- INT2 proposal
@pytest.mark.parametrize("D,dtype,T,lens", [(128, "f32", 3000, None), (64, "bf16", 3000, [3000, 1777]),
                                            (256, "bf16", 2500, [0, 2500]), (128, "bf16", 5000, None)])
def test_quantize_keys_int2_bitexact(D, dtype, T, lens):
    q, K, V, lens = make_inputs(D + T + 1, 2 if lens else 1, 4, 2, D, T, dtype, lens)
    K[0, 0, 5] = 0.0                    # an all-zero row
    K[0, 1, 7, :16] = 0.0               # values on the cell edge u = 0
    Kd = dev(K, dtype)
    ld = torch.from_numpy(lens).cuda()
    Kq2, sc = PB.quantize_keys_int2(Kd, seq_lens=ld)
    torch.cuda.synchronize()
    lv = unpack_int2(Kq2.cpu().numpy(), D)
    sc = sc.cpu().numpy()
    for b in range(K.shape[0]):
        n = lens[b]
        olv, osc = oracle.quantize_rows_int2(K[b, :, :n])
        assert np.array_equal(lv[b, :, :n], olv)
        assert np.array_equal(f32_bits(sc[b, :, :n]), f32_bits(osc))


@pytest.mark.parametrize("case", PROPOSE_CASES, ids=lambda c: f"D{c[0]}G{c[1]}a{c[3]}{c[4]}T{c[5]}kp{c[6]}")
@pytest.mark.parametrize("variant", ["random", "ties", "zero_q"])
def test_propose_int2_bitexact(case, variant):
    D, G, Hkv, agg, dtype, T, kp, lens = case
    Bn = len(lens) if lens else 1
    q, K, V, lens = make_inputs(seed_of(D, G, T, kp, variant, 2), Bn, G * Hkv, Hkv, D, T, dtype, lens,
                                ties=variant == "ties", zero_q=variant == "zero_q")
    ld = torch.from_numpy(lens).cuda()
    Kq2, sc = PB.quantize_keys_int2(dev(K, dtype), seq_lens=ld)
    scores = torch.zeros((Bn, Hkv, T), dtype=torch.float32, device="cuda")
    pool = PB.propose_int2(dev(q, dtype), Kq2, sc, kp, agg, seq_lens=ld, scores=scores)
    torch.cuda.synchronize()
    olv, osc = oracle.quantize_rows_int2(K)
    opool, oscores = oracle.propose(q, olv, osc, kp, seq_lens=lens, agg=agg, want_scores=True)
    gs = scores.cpu().numpy()
    for b in range(Bn):
        assert np.array_equal(f32_bits(gs[b, :, :lens[b]]), f32_bits(oscores[b, :, :lens[b]])), "scores differ"
    assert_pool_equal(pool.cpu().numpy(), opool)


def test_propose_large_candidate_set():
    """Every score equal over 262144 tokens: the threshold bin holds the whole context."""
    D, T, kp = 64, 262144, 65536
    rng = np.random.default_rng(9)
    K = np.tile(W.bf16_round(rng.standard_normal((1, 1, 1, D)).astype(np.float32)), (1, 1, T, 1))
    q = W.bf16_round(rng.standard_normal((1, 8, D)).astype(np.float32))
    Kq, sc, ld = gpu_quant(K, "bf16", np.array([T], np.int32))
    pool = PB.propose(dev(q, "bf16"), Kq, sc, kp, seq_lens=ld)
    torch.cuda.synchronize()
    assert pool.cpu().numpy()[0, 0].tolist() == list(range(kp))


# ------------------------------------------------------------------------------------- refine
REFINE_CASES = [
    # D, G, Hkv, agg, dtype, T, kp, kappa, lens
    (128, 4, 2, PB.AGG_SUM, "bf16", 6000, 2048, 512, None),
    (128, 1, 1, PB.AGG_SUM, "f32", 4096, 1024, 256, None),
    (64, 8, 2, PB.AGG_SUM, "bf16", 5000, 1000, 300, [5000, 2222]),
    (256, 4, 1, PB.AGG_MAX, "bf16", 3000, 1500, 700, None),
    (128, 3, 2, PB.AGG_MAX, "f32", 2000, 512, 100, None),
    (64, 16, 1, PB.AGG_SUM, "bf16", 3000, 600, 64, None),
    (256, 2, 1, PB.AGG_SUM, "f32", 1500, 900, 900, None),     # kappa = kp: static reuse
    (128, 4, 2, PB.AGG_SUM, "bf16", 1200, 2048, 1500, [1200, 0]),  # pool padding, empty sequence
    (128, 4, 1, PB.AGG_SUM, "bf16", 3000, 400, 1, None),        # kappa = 1
    (128, 1, 2, PB.AGG_SUM, "bf16", 4000, 1500, 400, None),      # one head per KV head
    (128, 2, 1, PB.AGG_MAX, "bf16", 4000, 1500, 400, None),
    (128, 3, 2, PB.AGG_SUM, "bf16", 4000, 1200, 333, None),      # G padded to 4
    (64, 8, 1, PB.AGG_MAX, "bf16", 3000, 1000, 250, None),       # MAX across two lane groups
    (128, 16, 1, PB.AGG_MAX, "bf16", 3000, 1000, 250, None),     # MAX across four lane groups
    (64, 4, 1, PB.AGG_SUM, "bf16", 20000, 10000, 3000, None),    # pool above one 8192-slot tile
    (128, 4, 1, PB.AGG_SUM, "bf16", 6000, 5000, 1000, None),     # one tile, clustered bin above 2048 keys
    (64, 4, 1, PB.AGG_MAX, "f32", 2000, 450, 100, None),         # clustered bin of 450 keys
    (128, 2, 1, PB.AGG_SUM, "bf16", 1000, 200, 50, None),        # clustered bin of 200 keys
    (128, 4, 2, PB.AGG_SUM, "bf16", 1200, 1024, 300, [1200, 0]), # head-dim split: empty sequence
    (256, 2, 1, PB.AGG_SUM, "bf16", 3000, 1200, 500, None),      # head-dim split: 32 pieces of D
    (128, 4, 1, PB.AGG_MAX, "bf16", 6000, 4096, 1024, None),     # head-dim split: most rows
    (64, 1, 1, PB.AGG_SUM, "f32", 3000, 800, 700, None),         # head-dim split: 4 values per lane
    (64, 16, 2, PB.AGG_SUM, "bf16", 1200, 1024, 300, [1200, 0]), # rank split (G > 8): empty sequence
    (128, 16, 1, PB.AGG_SUM, "f32", 3000, 2000, 1200, None),       # column halves of V, fp32
    (256, 4, 1, PB.AGG_SUM, "bf16", 4000, 3000, 2100, None),       # column quarters of 256-dim rows
    (128, 4, 1, PB.AGG_SUM, "bf16", 6000, 4096, 2048, None),       # head-dim split: most rows (2048)
    (64, 8, 1, PB.AGG_MAX, "f32", 4000, 3000, 1025, None),         # head-dim split: 2048-row variant
    (128, 2, 16, PB.AGG_SUM, "bf16", 2000, 1500, 700, None),       # head-dim split, 16-byte pieces (16 units)
    (128, 8, 16, PB.AGG_MAX, "bf16", 1500, 1024, 600, None),       # head-dim split, 16-byte pieces, 8 heads:
                                                                   # 64 sums per lane, the final sum on all threads
    (256, 8, 1, PB.AGG_MAX, "bf16", 9000, 8000, 4000, None),       # column quarters, two-level merge
    (128, 4, 1, PB.AGG_SUM, "bf16", 8000, 6000, 3000, None),       # column halves, two-level merge
    (64, 2, 16, PB.AGG_SUM, "bf16", 1500, 1024, 1024, [1500] * 8),  # 128 units: 512 ranks per workgroup
    (128, 4, 8, PB.AGG_MAX, "bf16", 2500, 1200, 1100,            # 64 units, 512 ranks, a partial slice,
     [2500, 1700, 0, 2500, 900, 2500, 2500, 1234]),                 # pools shorter than kappa, empty
]


@pytest.mark.parametrize("case", REFINE_CASES, ids=lambda c: f"D{c[0]}G{c[1]}a{c[3]}{c[4]}kp{c[6]}k{c[7]}")
@pytest.mark.parametrize("variant", ["random", "zero_q", "ties", "clustered", "dup"])
def test_refine_parity(case, variant):
    """'clustered' puts the whole pool in one or two top-12-bit score bins with exact scores, so
    the threshold is resolved from a long candidate list (direct counting up to 512 keys, the
    8-bit sub-histogram up to 2048, radix digits beyond) and the index sets must be identical."""
    D, G, Hkv, agg, dtype, T, kp, kappa, lens = case
    Bn = len(lens) if lens else 1
    q, K, V, lens = make_inputs(seed_of(D, G, T, kp, kappa, variant), Bn, G * Hkv, Hkv, D, T, dtype, lens,
                                zero_q=variant == "zero_q", ties=variant == "ties", clustered=variant == "clustered",
                                dup=37 if variant == "dup" else 0)
    rng = np.random.default_rng(kp + kappa)
    q0 = rnd(rng, q.shape, dtype)
    oKq, osc = oracle.quantize_rows(K)
    pool = oracle.propose(q0, oKq, osc, kp, seq_lens=lens)  # an oracle pool feeds both sides
    ld = torch.from_numpy(lens).cuda()
    out, idx, lse = PB.refine_attend(dev(q, dtype), dev(K, dtype), dev(V, dtype), torch.from_numpy(pool).cuda(),
                                     kappa, agg, seq_lens=ld)
    torch.cuda.synchronize()
    check_refine_batch(idx.cpu().numpy(), host(out), lse.cpu().numpy(), q, K, V, lens, pool, kappa, agg, dtype,
                       exact=variant in ("clustered", "dup"))
    if variant == "zero_q":  # every score ties: the lowest pool slots win
        gi = idx.cpu().numpy()
        for b in range(Bn):
            for g in range(Hkv):
                valid = pool[b, g][(pool[b, g] >= 0) & (pool[b, g] < lens[b])]
                n = min(kappa, len(valid))
                assert gi[b, g, :n].tolist() == valid[:n].tolist()


def test_refine_full_budget_is_dense():
    """kappa = kp = T_b: the refined layer reproduces dense attention (GPU sparse vs GPU dense vs oracle)."""
    D, G, Hkv, T = 128, 4, 2, 3000
    q, K, V, lens = make_inputs(77, 1, G * Hkv, Hkv, D, T, "bf16")
    pool = np.tile(np.arange(T, dtype=np.int32), (1, Hkv, 1))
    qd, Kd, Vd = dev(q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    out, idx, lse = PB.refine_attend(qd, Kd, Vd, torch.from_numpy(pool).cuda(), T)
    dout, dlse = PB.dense_ref(qd, Kd, Vd)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), pool)
    check_dense_batch(host(out), lse.cpu().numpy(), q, K, V, lens, "bf16")
    check_dense_batch(host(dout), dlse.cpu().numpy(), q, K, V, lens, "bf16")


@pytest.mark.parametrize("D,G,dtype,T,lens", [(128, 4, "bf16", 5000, [5000, 1234]), (64, 8, "f32", 3000, None),
                                             (256, 1, "bf16", 2000, [0, 2000]), (128, 3, "f32", 1000, None)])
def test_dense_parity(D, G, dtype, T, lens):
    Hkv = 2
    Bn = len(lens) if lens else 1
    q, K, V, lens = make_inputs(D * G + T, Bn, G * Hkv, Hkv, D, T, dtype, lens)
    out, lse = PB.dense_ref(dev(q, dtype), dev(K, dtype), dev(V, dtype), seq_lens=torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    check_dense_batch(host(out), lse.cpu().numpy(), q, K, V, lens, dtype)


# ------------------------------------------------------------------------------------- paged caches
def to_pages(X, P, rng, spare=3):
    """Logical [B, Hkv, T_max, ...] -> (pool [Hkv, S, ...], page table [B, max_pages] int32): every
    logical page of every sequence gets its own physical page, in shuffled order, with spare pages
    (zero) in between."""
    B, Hkv, T_max = X.shape[:3]
    max_pages = -(-T_max // P)
    n_pages = B * max_pages + spare
    table = rng.permutation(n_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    pool = np.zeros((Hkv, n_pages * P) + X.shape[3:], dtype=X.dtype)
    for b in range(B):
        for p in range(max_pages):
            t0, t1 = p * P, min((p + 1) * P, T_max)
            pool[:, table[b, p] * P: table[b, p] * P + (t1 - t0)] = X[b, :, t0:t1]
    return pool, table


PAGED_CASES = [
    # D, G, Hkv, agg, dtype, T, kp, kappa, lens, page size
    (128, 4, 2, PB.AGG_SUM, "bf16", 5000, 2048, 512, [5000, 3333], 16),
    (64, 8, 1, PB.AGG_SUM, "f32", 3000, 1000, 300, None, 1),
    (256, 1, 2, PB.AGG_MAX, "bf16", 2000, 700, 200, [0, 2000], 64),
    (128, 3, 2, PB.AGG_SUM, "bf16", 2600, 1200, 333, [2600, 77], 4096),
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=lambda c: f"D{c[0]}G{c[1]}a{c[3]}{c[4]}P{c[9]}")
@pytest.mark.parametrize("key_bits", [8, 2])
def test_paged_matches_contiguous(case, key_bits):
    """The paged calls on shuffled page pools give the contiguous calls' pools, scores, index sets,
    outputs and lse bit for bit, and the pools equal the oracle's."""
    D, G, Hkv, agg, dtype, T, kp, kappa, lens, P = case
    Bn = len(lens) if lens else 1
    q, K, V, lens = make_inputs(seed_of(D, G, T, P, key_bits), Bn, G * Hkv, Hkv, D, T, dtype, lens)
    rng = np.random.default_rng(P + key_bits)
    Kp, table = to_pages(K, P, rng)
    Vp, table2 = to_pages(V, P, np.random.default_rng(P + key_bits))
    assert np.array_equal(table, table2)
    ld = torch.from_numpy(lens).cuda()
    tab = torch.from_numpy(table).cuda()
    quant = PB.quantize_keys_int2 if key_bits == 2 else PB.quantize_keys
    qd = dev(q, dtype)
    # contiguous reference run
    Kq, sc = quant(dev(K, dtype), seq_lens=ld)
    prop = PB.propose_int2 if key_bits == 2 else PB.propose
    sc_c = torch.zeros((Bn, Hkv, T), dtype=torch.float32, device="cuda")
    pool_c = prop(qd, Kq, sc, kp, agg, seq_lens=ld, scores=sc_c)
    out_c, idx_c, lse_c = PB.refine_attend(qd, dev(K, dtype), dev(V, dtype), pool_c, kappa, agg, seq_lens=ld)
    # paged run: the pools are compressed as one [1, Hkv, S] cache
    Kq_p, sc_p = quant(dev(Kp, dtype)[None])
    sc_g = torch.zeros((Bn, Hkv, T), dtype=torch.float32, device="cuda")
    pool_p = PB.propose_paged(qd, Kq_p[0], sc_p[0], tab, P, kp, agg, key_bits=key_bits, T_max=T, seq_lens=ld,
                              scores=sc_g)
    out_p, idx_p, lse_p = PB.refine_attend_paged(qd, dev(Kp, dtype), dev(Vp, dtype), tab, P, pool_p, kappa, agg,
                                                 T_max=T, seq_lens=ld)
    torch.cuda.synchronize()
    assert torch.equal(pool_p, pool_c)
    for b in range(Bn):
        n = int(lens[b])
        assert torch.equal(sc_g[b, :, :n], sc_c[b, :, :n])
    assert torch.equal(idx_p, idx_c)
    assert torch.equal(out_p, out_c)
    assert torch.equal(lse_p, lse_c)
    lv, osc = (oracle.quantize_rows_int2 if key_bits == 2 else oracle.quantize_rows)(K)
    opool = oracle.propose(q, lv, osc, kp, seq_lens=lens, agg=agg)
    assert_pool_equal(pool_p.cpu().numpy(), opool)
    # the paged refined layer against the oracle on the logical caches (not only against the
    # contiguous GPU path)
    check_refine_batch(idx_p.cpu().numpy(), host(out_p), lse_p.cpu().numpy(), q, K, V, lens, opool, kappa, agg,
                       dtype)


# ------------------------------------------------------------------ proposal on CU-filling grids
# Shapes whose 4096-token work items give at least 256 scan workgroups (one per CU), where the
# scan runs one 1024-thread workgroup per CU with batches claimed by its waves: ragged tails,
# MAX aggregation, two work items per workgroup, INT2 keys, fp32 queries, paged caches (pages of
# 4 tokens are smaller than a wave-load and take the 256-thread scan at the same grid size) and a
# T_max that is no multiple of the work item (the last work item is partial and is a workgroup's
# second one).
WIDE_CASES = [
    # D, G, Hkv, agg, dtype, T, kp, lens, key bits, page size (0: contiguous)
    (128, 4, 8, PB.AGG_SUM, "bf16", 65536, 4096, [65536, 50001], 8, 0),
    (128, 3, 8, PB.AGG_MAX, "bf16", 65536, 2048, None, 8, 0),
    (64, 1, 8, PB.AGG_SUM, "f32", 131072, 1000, [131072, 77777], 8, 0),
    (256, 2, 8, PB.AGG_SUM, "bf16", 65536, 3000, [4095, 65536], 2, 0),
    (128, 4, 8, PB.AGG_MAX, "bf16", 65536, 1500, [65000, 65536], 2, 0),
    (128, 4, 8, PB.AGG_SUM, "bf16", 65536, 4096, [65536, 40000], 8, 16),
    (128, 4, 8, PB.AGG_SUM, "bf16", 65536, 2048, [65536, 33333], 2, 64),
    (128, 4, 8, PB.AGG_SUM, "bf16", 65536, 2048, [65536, 30001], 8, 4),
    (128, 4, 8, PB.AGG_SUM, "bf16", 65541, 2048, [65541, 61234], 8, 0),  # T_max not a multiple of 4
    (128, 4, 8, PB.AGG_SUM, "bf16", 65541, 2048, [65541, 4097], 2, 0),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: f"D{c[0]}G{c[1]}a{c[3]}{c[4]}T{c[5]}kb{c[8]}P{c[9]}")
def test_propose_cu_filling_grid(case):
    D, G, Hkv, agg, dtype, T, kp, lens, key_bits, P = case
    Bn = len(lens) if lens else 2
    rng = np.random.default_rng(seed_of(D, G, T, kp, key_bits, P))
    q = rnd(rng, (Bn, G * Hkv, D), dtype)
    K = rnd(rng, (Bn, Hkv, T, D), dtype)
    lens = np.full(Bn, T, np.int32) if lens is None else np.asarray(lens, np.int32)
    for b in range(Bn):
        K[b, :, lens[b]:] = 0.0
    ld = torch.from_numpy(lens).cuda()
    quant = PB.quantize_keys_int2 if key_bits == 2 else PB.quantize_keys
    qd = dev(q, dtype)
    scores = torch.zeros((Bn, Hkv, T), dtype=torch.float32, device="cuda")
    if P:
        Kp, table = to_pages(K, P, rng)
        Kq_p, sc_p = quant(dev(Kp, dtype)[None])
        pool = PB.propose_paged(qd, Kq_p[0], sc_p[0], torch.from_numpy(table).cuda(), P, kp, agg,
                                key_bits=key_bits, T_max=T, seq_lens=ld, scores=scores)
    else:
        Kq, sc = quant(dev(K, dtype), seq_lens=ld)
        prop = PB.propose_int2 if key_bits == 2 else PB.propose
        pool = prop(qd, Kq, sc, kp, agg, seq_lens=ld, scores=scores)
    torch.cuda.synchronize()
    lv, osc = (oracle.quantize_rows_int2 if key_bits == 2 else oracle.quantize_rows)(K)
    opool, oscores = oracle.propose(q, lv, osc, kp, seq_lens=lens, agg=agg, want_scores=True)
    gs = scores.cpu().numpy()
    for b in range(Bn):
        assert np.array_equal(f32_bits(gs[b, :, :lens[b]]), f32_bits(oscores[b, :, :lens[b]])), "scores differ"
    assert_pool_equal(pool.cpu().numpy(), opool)


# ------------------------------------------------------------------------------------- whole steps
def run_step_gpu(w, kp, kappa, agg=PB.AGG_SUM, key_bits=8):
    from token_level_sparse_prism_amd.step import LayerInputs, PrismStep
    c = w.cfg
    ld = torch.from_numpy(w.seq_lens).cuda()
    quant = PB.quantize_keys_int2 if key_bits == 2 else PB.quantize_keys
    Kq, sc = quant(dev(w.K[0], c.dtype), seq_lens=ld)
    layers = [LayerInputs(dev(w.q[l], c.dtype), dev(w.K[l], c.dtype), dev(w.V[l], c.dtype))
              for l in range(1, w.layers)]
    step = PrismStep(dev(w.q[0], c.dtype), Kq, sc, layers, kp, kappa, agg, seq_lens=ld, key_bits=key_bits)
    pool, idx, out, lse = step()
    torch.cuda.synchronize()
    return step, Kq, sc


@pytest.mark.parametrize("name,overrides", [("cfg1", {}), ("cfg2", {"B": 1, "T": 32768}),
                                            ("cfg4", {"B": 2, "T": 24576, "ragged": (8192, 24576), "n_refined": 2}),
                                            ("cfg5_D64_k512_r4", {"T": 16384}), ("cfg5_D256_k512_r2", {"T": 8192})])
def test_config_step_parity(name, overrides):
    c = W.CONFIGS[name].with_(**overrides)
    w = W.generate(c)
    step, Kq, sc = run_step_gpu(w, c.kp, c.kappa)
    oKq, osc = oracle.quantize_rows(w.K[0])
    for b in range(c.B):
        n = w.seq_lens[b]
        assert np.array_equal(Kq.cpu().numpy()[b, :, :n], oKq[b, :, :n])
    opool = oracle.propose(w.q[0], oKq, osc, c.kp, seq_lens=w.seq_lens)
    assert_pool_equal(step.pool.cpu().numpy(), opool)
    for l in range(1, w.layers):
        check_refine_batch(step.idx[l - 1].cpu().numpy(), host(step.out[l - 1]), step.lse[l - 1].cpu().numpy(),
                           w.q[l], w.K[l], w.V[l], w.seq_lens, opool, c.kappa, PB.AGG_SUM, c.dtype)
        # planted recovery: each refined layer's salient tokens that the pool holds are selected
        for b in range(c.B):
            for g in range(c.Hkv):
                S0, Sl = w.salient[(b, g)]
                inpool = Sl[l - 1][np.isin(Sl[l - 1], opool[b, g])]
                assert np.isin(inpool, step.idx[l - 1].cpu().numpy()[b, g]).all()
                assert np.isin(S0, opool[b, g]).all()


def test_determinism_and_workspace_reuse():
    """Ten steps with the same workspaces give bit-identical pools, index sets and outputs."""
    c = W.CONFIGS["cfg2"].with_(B=1, Hkv=4, Hq=16, T=20000)
    w = W.generate(c)
    step, _, _ = run_step_gpu(w, c.kp, c.kappa)
    ref = [step.pool.clone()] + [t.clone() for t in step.idx] + [t.clone() for t in step.out]
    for _ in range(10):
        step()
        torch.cuda.synchronize()
        cur = [step.pool] + list(step.idx) + list(step.out)
        for a, b in zip(ref, cur):
            assert torch.equal(a, b)


def test_split_independence():
    """The same unit alone and inside a batch of 128 units: the scan splits its 32 chunks over 32
    workgroups alone and over 8 workgroups (4 chunks each) in the batch, and the attention takes
    128 ranks per workgroup alone and 256 in the batch (the batch has more workgroups than CUs).
    Pools and index sets of that unit are bit-identical, outputs and lse within the bf16
    tolerance (P10)."""
    D, G, T, kp, kappa = 64, 2, 32768, 4096, 1024
    Bn, Hkv = 8, 16
    q, K, V, lens = make_inputs(31337, Bn, G * Hkv, Hkv, D, T, "bf16")
    ld = torch.from_numpy(lens).cuda()
    Kq, sc = PB.quantize_keys(dev(K, "bf16"), seq_lens=ld)
    pool_b = PB.propose(dev(q, "bf16"), Kq, sc, kp, seq_lens=ld)
    out_b, idx_b, lse_b = PB.refine_attend(dev(q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), pool_b, kappa, seq_lens=ld)
    b, g = 5, 11
    q1 = np.ascontiguousarray(q[b:b + 1, g * G:(g + 1) * G])
    K1, V1 = np.ascontiguousarray(K[b:b + 1, g:g + 1]), np.ascontiguousarray(V[b:b + 1, g:g + 1])
    ld1 = torch.from_numpy(lens[b:b + 1]).cuda()
    Kq1, sc1 = PB.quantize_keys(dev(K1, "bf16"), seq_lens=ld1)
    pool_1 = PB.propose(dev(q1, "bf16"), Kq1, sc1, kp, seq_lens=ld1)
    out_1, idx_1, lse_1 = PB.refine_attend(dev(q1, "bf16"), dev(K1, "bf16"), dev(V1, "bf16"), pool_1, kappa,
                                           seq_lens=ld1)
    torch.cuda.synchronize()
    assert torch.equal(pool_1[0, 0], pool_b[b, g])
    assert torch.equal(idx_1[0, 0], idx_b[b, g])
    d_out = (out_1[0].float() - out_b[b, g * G:(g + 1) * G].float()).abs().max().item()
    d_lse = (lse_1[0] - lse_b[b, g * G:(g + 1) * G]).abs().max().item()
    assert d_out <= 2e-2 and d_lse <= 1e-4, (d_out, d_lse)


def test_graph_replay_int2():
    """A HIP graph of a whole step with INT2 proposal keys replays to the eager step bit for bit."""
    c = W.CONFIGS["cfg2"].with_(B=1, Hkv=2, Hq=8, T=12000)
    w = W.generate(c)
    step, _, _ = run_step_gpu(w, c.kp, c.kappa, key_bits=2)
    ref = [step.pool.clone()] + [t.clone() for t in step.idx] + [t.clone() for t in step.out]
    graph = step.capture()
    for i in range(3):
        for t in [step.pool] + list(step.idx) + list(step.out):
            t.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, [step.pool] + list(step.idx) + list(step.out)):
            assert torch.equal(a, b), f"replay {i}"


def test_full_size_128k_all_units():
    """The 128K-context workload at full size, in the launch configuration the benchmark times:
    every unit's pool bit for bit and every unit's refined layers in full against the oracle."""
    c = W.CONFIGS["cfg3"]
    w = W.generate(c)
    step, Kq, sc = run_step_gpu(w, c.kp, c.kappa)
    oKq, osc = oracle.quantize_rows(w.K[0])
    assert np.array_equal(Kq.cpu().numpy(), oKq)
    assert np.array_equal(f32_bits(sc.cpu().numpy()), f32_bits(osc))
    opool = oracle.propose(w.q[0], oKq, osc, c.kp, seq_lens=w.seq_lens)
    gpool = step.pool.cpu().numpy()
    assert_pool_equal(gpool, opool)
    for l in range(1, w.layers):
        gidx = step.idx[l - 1].cpu().numpy()
        for g in range(c.Hkv):
            assert set(gidx[0, g].tolist()) <= set(gpool[0, g].tolist())
        check_refine_batch(gidx, host(step.out[l - 1]), step.lse[l - 1].cpu().numpy(), w.q[l], w.K[l], w.V[l],
                           w.seq_lens, opool, c.kappa, PB.AGG_SUM, c.dtype)


@pytest.mark.parametrize("name", ["cfg5_D256_k8192_r8", "cfg5_D64_k2048_r4"])
def test_full_size_262k_single_unit(name):
    """The 262144-token stress workloads at full size (Student-t keys, 8 query heads on one KV
    head): the pool bit for bit, and every refined layer in full against the oracle.  At
    kp = 65536 the refine selection runs over eight 8192-slot tiles."""
    c = W.CONFIGS[name]
    w = W.generate(c)
    step, Kq, sc = run_step_gpu(w, c.kp, c.kappa)
    oKq, osc = oracle.quantize_rows(w.K[0])
    assert np.array_equal(Kq.cpu().numpy(), oKq)
    opool = oracle.propose(w.q[0], oKq, osc, c.kp, seq_lens=w.seq_lens)
    assert_pool_equal(step.pool.cpu().numpy(), opool)
    for l in range(1, w.layers):
        check_refine_batch(step.idx[l - 1].cpu().numpy(), host(step.out[l - 1]), step.lse[l - 1].cpu().numpy(),
                           w.q[l], w.K[l], w.V[l], w.seq_lens, opool, c.kappa, PB.AGG_SUM, c.dtype)


def test_full_size_cfg2_all_units():
    """The 32K-context batch-4 workload at full size: every unit's pool bit for bit, and every
    unit's refined layers in full."""
    c = W.CONFIGS["cfg2"]
    w = W.generate(c)
    step, Kq, sc = run_step_gpu(w, c.kp, c.kappa)
    oKq, osc = oracle.quantize_rows(w.K[0])
    opool = oracle.propose(w.q[0], oKq, osc, c.kp, seq_lens=w.seq_lens)
    assert_pool_equal(step.pool.cpu().numpy(), opool)
    for l in range(1, w.layers):
        check_refine_batch(step.idx[l - 1].cpu().numpy(), host(step.out[l - 1]), step.lse[l - 1].cpu().numpy(),
                           w.q[l], w.K[l], w.V[l], w.seq_lens, opool, c.kappa, PB.AGG_SUM, c.dtype)


def test_full_size_128k_int2():
    """The 128K-context workload with INT2 proposal keys: the packed codes and scales, every
    unit's pool bit for bit, every unit's refined layers in full, and the anchor's unshifted
    planted tokens in every pool."""
    c = W.CONFIGS["cfg3"]
    w = W.generate(c)
    step, Kq2, sc = run_step_gpu(w, c.kp, c.kappa, key_bits=2)
    olv, osc = oracle.quantize_rows_int2(w.K[0])
    assert np.array_equal(unpack_int2(Kq2.cpu().numpy(), c.D), olv)
    assert np.array_equal(f32_bits(sc.cpu().numpy()), f32_bits(osc))
    opool = oracle.propose(w.q[0], olv, osc, c.kp, seq_lens=w.seq_lens)
    gpool = step.pool.cpu().numpy()
    assert_pool_equal(gpool, opool)
    for g in range(c.Hkv):
        assert np.isin(w.salient[(0, g)][0], gpool[0, g]).all()
    for l in range(1, w.layers):
        check_refine_batch(step.idx[l - 1].cpu().numpy(), host(step.out[l - 1]), step.lse[l - 1].cpu().numpy(),
                           w.q[l], w.K[l], w.V[l], w.seq_lens, opool, c.kappa, PB.AGG_SUM, c.dtype)


def test_graph_replay_matches_eager():
    """A HIP graph of one whole step, replayed several times with eager work in between, gives the
    eager step's pools, index sets and outputs bit for bit every time."""
    c = W.CONFIGS["cfg2"].with_(B=1, Hkv=2, Hq=8, T=12000)
    w = W.generate(c)
    step, _, _ = run_step_gpu(w, c.kp, c.kappa)
    ref = [step.pool.clone()] + [t.clone() for t in step.idx] + [t.clone() for t in step.out]
    graph = step.capture()
    for i in range(5):
        for t in [step.pool] + list(step.idx) + list(step.out):
            t.fill_(7)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        cur = [step.pool] + list(step.idx) + list(step.out)
        for a, b in zip(ref, cur):
            assert torch.equal(a, b), f"replay {i}"


@pytest.mark.timeout(900)
def test_full_shape_cfg4():
    """The batched long-context workload at its real shape (8 sequences of 16K-128K tokens from
    the seed-4 draw, 64 query / 8 KV heads, 7 refined layers), generated one layer at a time
    straight to the device as the benchmark does: every unit's pool bit for bit (each unit's
    anchor keys regenerated on the host), and the refined layers of 8 units against the oracle
    (units spread over every sequence, the shortest and longest among them)."""
    c = W.CONFIGS["cfg4"]
    lens = c.lengths()
    ld = torch.from_numpy(lens).cuda()
    from token_level_sparse_prism_amd.step import LayerInputs, PrismStep
    q_host, layers = [], []
    sample = [(b, (3 * b + 1) % c.Hkv) for b in range(c.B)]
    kept = {}
    Kq = sc = q0 = None
    for l in range(c.n_refined + 1):
        wl = W.generate(c, layers=[l])
        q_host.append(wl.q[0])
        if l == 0:
            K0 = dev(wl.K[0], c.dtype)
            Kq, sc = PB.quantize_keys(K0, seq_lens=ld)
            q0 = dev(wl.q[0], c.dtype)
            del K0
        else:
            layers.append(LayerInputs(dev(wl.q[0], c.dtype), dev(wl.K[0], c.dtype), dev(wl.V[0], c.dtype)))
            for (b, g) in sample:
                kept[(l, b, g)] = (wl.K[0][b, g].copy(), wl.V[0][b, g].copy())
        del wl
        torch.cuda.synchronize()
    step = PrismStep(q0, Kq, sc, layers, c.kp, c.kappa, seq_lens=ld)
    step()
    torch.cuda.synchronize()
    gpool = step.pool.cpu().numpy()
    gidx = [t.cpu().numpy() for t in step.idx]
    gout = [host(t) for t in step.out]
    glse = [t.cpu().numpy() for t in step.lse]
    G = c.G
    for b in range(c.B):
        T_b = int(lens[b])
        for g in range(c.Hkv):
            K0, _ = W.unit_tensors(c, b, g, 0, q_host[0], T_b, want_v=False)
            oKq, osc = oracle.quantize_rows(K0)
            opool, _ = oracle.propose_unit(q_host[0][b, g * G:(g + 1) * G], oKq, osc, T_b, c.kp)
            assert_pool_equal(gpool[b, g][None], opool[None])
            if (b, g) not in sample:
                continue
            for l in range(1, c.n_refined + 1):
                Kl, Vl = kept[(l, b, g)]
                from tests.parity import check_refine_unit
                check_refine_unit(gidx[l - 1][b, g], gout[l - 1][b, g * G:(g + 1) * G],
                                  glse[l - 1][b, g * G:(g + 1) * G], q_host[l][b, g * G:(g + 1) * G], Kl, Vl, T_b,
                                  opool, c.kappa, PB.AGG_SUM, c.dtype, where=f"layer {l} unit ({b},{g})")


def test_shared_workspace_propose_refine():
    """One zero-filled workspace, sized for the larger of the two ops, serves a proposal, the
    refined layers, the next proposal and so on: the results equal those of separate workspaces
    (the refine layout keeps its data clear of the proposal's zero-on-entry histogram, and pool
    scoring zeroes the attention's arrival counters itself)."""
    c = W.CONFIGS["cfg2"].with_(B=2, T=20000, seq_lens=(20000, 11111))
    w = W.generate(c)
    ld = torch.from_numpy(w.seq_lens).cuda()
    Kq, sc = PB.quantize_keys(dev(w.K[0], c.dtype), seq_lens=ld)
    q0 = dev(w.q[0], c.dtype)
    layers = [(dev(w.q[l], c.dtype), dev(w.K[l], c.dtype), dev(w.V[l], c.dtype)) for l in range(1, w.layers)]
    shp = PB.make_shape(q0, Kq, ld)
    nbytes = max(PB.workspace_bytes(PB.OP_PROPOSE, shp, c.kp), PB.workspace_bytes(PB.OP_REFINE, shp, c.kp, c.kappa))
    shared = PB.new_workspace_bytes(nbytes)
    ref_pool = PB.propose(q0, Kq, sc, c.kp, seq_lens=ld)
    ref = [PB.refine_attend(q, K, V, ref_pool, c.kappa, seq_lens=ld) for q, K, V in layers]
    torch.cuda.synchronize()
    for rep in range(3):
        pool = PB.propose(q0, Kq, sc, c.kp, seq_lens=ld, ws=shared)
        outs = [PB.refine_attend(q, K, V, pool, c.kappa, seq_lens=ld, ws=shared) for q, K, V in layers]
        torch.cuda.synchronize()
        assert torch.equal(pool, ref_pool), f"pass {rep}: pool"
        for (o, i, s_), (ro, ri, rs) in zip(outs, ref):
            assert torch.equal(i, ri) and torch.equal(o, ro) and torch.equal(s_, rs), f"pass {rep}: refine"


@pytest.mark.parametrize("name,overrides", [("cfg2", {"B": 2, "T": 32768}), ("cfg3", {"Hkv": 2, "Hq": 8})])
def test_anchor_attention_step(name, overrides):
    """The step variant in which the anchor layer also attends: refine_attend on layer 0's exact
    K and V with the pool it proposed.  Its index set and outputs against the oracle's refine on
    layer 0 with the oracle's pool, and the refined layers unchanged by it."""
    from token_level_sparse_prism_amd.step import LayerInputs, PrismStep
    c = W.CONFIGS[name].with_(anchor_v=True, **overrides)
    w = W.generate(c)
    ld = torch.from_numpy(w.seq_lens).cuda()
    K0 = dev(w.K[0], c.dtype)
    Kq, sc = PB.quantize_keys(K0, seq_lens=ld)
    q0 = dev(w.q[0], c.dtype)
    layers = [LayerInputs(dev(w.q[l], c.dtype), dev(w.K[l], c.dtype), dev(w.V[l], c.dtype))
              for l in range(1, w.layers)]
    step = PrismStep(q0, Kq, sc, layers, c.kp, c.kappa, seq_lens=ld,
                     anchor=LayerInputs(q0, K0, dev(w.V[0], c.dtype)))
    plain = PrismStep(q0, Kq, sc, layers, c.kp, c.kappa, seq_lens=ld)
    step()
    torch.cuda.synchronize()
    anchor = (step.idx_anchor.cpu().numpy(), host(step.out_anchor), step.lse_anchor.cpu().numpy())
    refined = [(t.clone(), o.clone()) for t, o in zip(step.idx, step.out)]
    plain()
    torch.cuda.synchronize()
    oKq, osc = oracle.quantize_rows(w.K[0])
    opool = oracle.propose(w.q[0], oKq, osc, c.kp, seq_lens=w.seq_lens)
    assert_pool_equal(step.pool.cpu().numpy(), opool)
    check_refine_batch(anchor[0], anchor[1], anchor[2], w.q[0], w.K[0], w.V[0], w.seq_lens, opool, c.kappa,
                       PB.AGG_SUM, c.dtype)
    for b in range(c.B):  # the anchor's own planted tokens are what its attention selects
        for g in range(c.Hkv):
            assert np.isin(w.salient[(b, g)][0], anchor[0][b, g]).all()
    for (i, o), i2, o2 in zip(refined, plain.idx, plain.out):
        assert torch.equal(i, i2) and torch.equal(o, o2)
