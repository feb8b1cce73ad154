"""Comparison helpers for the GPU parity tests: the HIP path (through the C ABI) against the CPU
oracle, with the bars of the hot path: bit-exact keys, scores and pools; refined index sets equal
up to near-ties of the oracle's score; attention outputs within a dtype tolerance, evaluated on
the GPU's own index set."""
import math

import numpy as np
import torch

import oracle

OUT_TOL = {"bf16": 2e-2, "f32": 1e-4}
LSE_TOL = {"bf16": 1e-3, "f32": 1e-4}
TIE_REL = 1e-3


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def host(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def unpack_int2(Kq2, D):
    """Levels {-3,-1,1,3} [..., D] of packed 2-bit keys [..., D/4] bytes: 32-bit word w of a row
    (little endian) holds dim 16w + 4j + i in bits 8i + 2j .. 8i + 2j + 1, code b, level 2b - 3."""
    a = np.ascontiguousarray(Kq2, dtype=np.uint8)
    words = a.reshape(a.shape[:-1] + (D // 16, 4)).view(np.uint32)[..., 0]  # [..., D/16]
    out = np.empty(a.shape[:-1] + (D // 16, 4, 4), dtype=np.int8)  # [..., w, j, i]
    for j in range(4):
        for i in range(4):
            out[..., j, i] = ((words >> (8 * i + 2 * j)) & 3).astype(np.int8) * 2 - 3
    return out.reshape(a.shape[:-1] + (D,))


def assert_pool_equal(gpu_pool, orc_pool):
    g, o = np.asarray(gpu_pool), np.asarray(orc_pool)
    assert g.shape == o.shape
    if not np.array_equal(g, o):
        bad = np.argwhere(np.any(g != o, axis=-1))
        u = tuple(bad[0])
        gi, oi = g[u], o[u]
        raise AssertionError(f"pool mismatch at unit {u}: gpu-only {sorted(set(gi) - set(oi))[:10]} "
                             f"oracle-only {sorted(set(oi) - set(gi))[:10]}")


def check_refine_unit(gpu_idx, gpu_out, gpu_lse, q_group, K, V, T_b, pool, kappa, agg, dtype, where="", exact=False):
    """One unit: tie-banded index parity (identical sets when `exact`: scores that both sides
    compute without rounding), then attention on the GPU's own selection."""
    r = oracle.refine_unit(q_group, K, V, T_b, pool, kappa, agg)
    gi = np.asarray(gpu_idx, dtype=np.int64)
    oi = r["idx"].astype(np.int64)
    nv = int((oi >= 0).sum())
    assert int((gi >= 0).sum()) == nv, f"{where}: |idx| {int((gi >= 0).sum())} vs {nv}"
    assert np.all(gi[nv:] == -1) and np.all(np.diff(gi[:nv]) > 0), f"{where}: idx not ascending/-1 padded"
    valid_pool = set(int(t) for t in pool if 0 <= t < T_b)
    gs, os_ = set(gi[:nv].tolist()), set(oi[:nv].tolist())
    assert gs <= valid_pool, f"{where}: idx not inside the pool"
    diff = gs ^ os_
    assert not (exact and diff), f"{where}: idx differs from the oracle's: {sorted(diff)[:10]}"
    if diff:
        S_of = {int(t): r["S"][j] for j, t in enumerate(pool) if 0 <= t < T_b}
        Ssorted = sorted(S_of.values(), reverse=True)
        s_star = Ssorted[nv - 1]
        band = TIE_REL * max(abs(s_star), 1e-6 * max(abs(x) for x in Ssorted))
        for t in diff:
            assert abs(S_of[t] - s_star) <= band, f"{where}: token {t} S={S_of[t]} vs kth {s_star}"
    out_g, lse_g = oracle.attend_unit(q_group, K, V, T_b, gi[:nv])
    err = np.abs(np.asarray(gpu_out, np.float64) - out_g).max() if nv else np.abs(gpu_out).max()
    assert err <= OUT_TOL[dtype], f"{where}: out err {err}"
    if gpu_lse is not None:
        if nv == 0:
            assert np.all(np.isneginf(gpu_lse)), f"{where}: empty selection lse"
        else:
            lerr = np.abs(np.asarray(gpu_lse, np.float64) - lse_g).max()
            assert lerr <= LSE_TOL[dtype], f"{where}: lse err {lerr}"
    if gs == os_ and nv:
        err2 = np.abs(np.asarray(gpu_out, np.float64) - r["out"]).max()
        assert err2 <= OUT_TOL[dtype], f"{where}: out err vs oracle selection {err2}"
    return len(diff)


def check_refine_batch(idx, out, lse, q, K, V, lens, pool, kappa, agg, dtype, units=None, exact=False):
    """Every (or the listed) unit of a batched refine call."""
    Bn, Hkv = pool.shape[:2]
    G = q.shape[1] // Hkv
    nties = 0
    for b in range(Bn):
        for g in range(Hkv):
            if units is not None and (b, g) not in units:
                continue
            h0 = g * G
            nties += check_refine_unit(idx[b, g], out[b, h0:h0 + G], None if lse is None else lse[b, h0:h0 + G],
                                       q[b, h0:h0 + G], K[b, g], V[b, g], int(lens[b]), pool[b, g], kappa, agg,
                                       dtype, where=f"unit ({b},{g})", exact=exact)
    return nties


def check_dense_batch(out, lse, q, K, V, lens, dtype):
    o, l = oracle.dense(q, K, V, seq_lens=lens)
    err = np.abs(np.asarray(out, np.float64) - o).max()
    assert err <= OUT_TOL[dtype], f"dense out err {err}"
    fin = np.isfinite(l)
    assert np.all(np.isneginf(np.asarray(lse)[~fin]))
    lerr = np.abs(np.asarray(lse, np.float64)[fin] - l[fin]).max() if fin.any() else 0.0
    assert lerr <= LSE_TOL[dtype], f"dense lse err {lerr}"


def sm_scale(D):
    return 1.0 / math.sqrt(D)
