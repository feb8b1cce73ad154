"""Seeded synthetic GQA decode workloads for the Prism decode hot path.

This module only MAKES inputs: it holds none of the method's arithmetic
(no quantization, no scoring, no selection, no attention).  Both the CPU
oracle side (tests) and the GPU side (tests, benchmark) draw their inputs
here.

Shapes and structure follow the Prism Attention page (paperpeel, arXiv
2610.22985): contexts up to 128K tokens and sparse budget kappa = 2048 with
expansion factor rho in {2, 4} (Sec. 5.1 Implementation Details), one
proposal layer per group of four (Sec. 5.3 accuracy-efficiency trade-off,
Table 3 caption), and a localized inter-layer shift of salient tokens
(Sec. 1, Sec. 3, Figure 2 notes: a shifted token sits just outside the
anchor's top set).  RoPE uses geometric frequencies theta_j = base^(-2j/D)
(Spectral Structure of RoPE paragraph of the second "Prism" page, arXiv
2602.08426), only to exercise a realistic data path.

Recipe, per layer l (0 = proposal/anchor, 1..L = refined) and unit (b, g):
  q_l [B,Hq,D] ~ N(0,1), rotated at position T_b - 1;
  K_l [B,Hkv,T_max,D] ~ N(0,1) (Student-t nu=3 when key_dist='student_t3'),
      rotated at position t; rows t >= T_b are zero;
  V_l ~ N(0,1) (refined layers; the anchor's V only when asked);
  salient set S_0 (n_salient positions); each refined layer's S_l replaces
      shift_frac of S_0 by s + delta, delta uniform in +-[1, shift_max];
  planted rows: K_l[t] = amp * sqrt(D) * u_{l,g} for t in S_l, where u is
      the unit vector of the sum of the group's queries;
  each shifted target p gets, at the anchor, K_0[p] = z_r * u_{0,g} with
      z_r the standard-normal quantile of a rank r ~ U[kappa, 3*kappa) among
      T_b noise tokens (analytic, no scoring), so that static reuse misses
      it and a pool of 4*kappa holds it;
  bf16 configs round every value to bf16 (round to nearest even).
Every random draw is keyed by (config seed, layer, tensor, b, head), so one
unit can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import math
import os
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from statistics import NormalDist
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

_Q, _K, _V, _SAL, _SHIFT, _RANK, _LENS = 1, 2, 3, 4, 5, 6, 7


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int                       # T_max, allocated capacity
    dtype: str                   # 'f32' or 'bf16'
    n_refined: int
    kp: int
    kappa: int
    rope_base: Optional[float]
    n_salient: int
    shift_frac: float = 0.2
    shift_max: int = 64
    amp: float = 4.0
    key_dist: str = "normal"     # or 'student_t3'
    ragged: Optional[Tuple[int, int]] = None  # (lo, hi) for per-sequence lengths
    seq_lens: Optional[Tuple[int, ...]] = None  # explicit lengths (override)
    anchor_v: bool = False

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def units(self) -> int:
        return self.B * self.Hkv

    def lengths(self) -> np.ndarray:
        if self.seq_lens is not None:
            return np.asarray(self.seq_lens, dtype=np.int32)
        if self.ragged is not None:
            lo, hi = self.ragged
            rng = np.random.default_rng(self.seed)
            return rng.integers(lo, hi, size=self.B, endpoint=True).astype(np.int32)
        return np.full(self.B, self.T, dtype=np.int32)

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def _cfg5(D: int, kappa: int, rho: int) -> Config:
    return Config(name=f"cfg5_D{D}_k{kappa}_r{rho}", seed=5, B=1, Hq=8, Hkv=1, D=D, T=262144,
                  dtype="bf16", n_refined=3, kp=rho * kappa, kappa=kappa, rope_base=None,
                  n_salient=max(kappa // 8, 1), key_dist="student_t3")


# The five workloads.  Config 3 is the 128K-context headline case.
CONFIGS: Dict[str, Config] = {
    "cfg1": Config(name="cfg1", seed=1, B=1, Hq=1, Hkv=1, D=128, T=4096, dtype="f32",
                   n_refined=1, kp=1024, kappa=256, rope_base=None, n_salient=16,
                   shift_frac=0.0),
    "cfg2": Config(name="cfg2", seed=2, B=4, Hq=32, Hkv=8, D=128, T=32768, dtype="bf16",
                   n_refined=3, kp=4096, kappa=2048, rope_base=500000.0, n_salient=256),
    "cfg3": Config(name="cfg3", seed=3, B=1, Hq=32, Hkv=8, D=128, T=131072, dtype="bf16",
                   n_refined=3, kp=8192, kappa=2048, rope_base=1e6, n_salient=256),
    "cfg4": Config(name="cfg4", seed=4, B=8, Hq=64, Hkv=8, D=128, T=131072, dtype="bf16",
                   n_refined=7, kp=8192, kappa=2048, rope_base=1e6, n_salient=256,
                   ragged=(16384, 131072)),
}
for _D in (64, 256):
    for _kappa in (512, 2048, 8192):
        for _rho in (1, 2, 4, 8):
            _c = _cfg5(_D, _kappa, _rho)
            CONFIGS[_c.name] = _c


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000))
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit pattern (uint16) of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


_ROPE_CACHE: Dict[Tuple[int, int, float], Tuple[np.ndarray, np.ndarray]] = {}
_ROPE_LOCK = threading.Lock()


def _rope_tables(n: int, D: int, base: float) -> Tuple[np.ndarray, np.ndarray]:
    key = (n, D, base)
    with _ROPE_LOCK:
        tab = _ROPE_CACHE.get(key)
        if tab is None:
            j = np.arange(D // 2, dtype=np.float64)
            theta = base ** (-2.0 * j / D)
            ang = np.arange(n, dtype=np.float64)[:, None] * theta[None, :]
            tab = (np.cos(ang), np.sin(ang))
            _ROPE_CACHE.clear()
            _ROPE_CACHE[key] = tab
    return tab


def rope_rotate(x: np.ndarray, positions: np.ndarray, base: float, cos_sin=None) -> np.ndarray:
    """Rotate-half RoPE: pairs (i, i + D/2) turned by position * base^(-2i/D). float64 result."""
    D = x.shape[-1]
    h = D // 2
    if cos_sin is None:
        j = np.arange(h, dtype=np.float64)
        theta = base ** (-2.0 * j / D)
        ang = positions.astype(np.float64)[:, None] * theta[None, :]
        c, s = np.cos(ang), np.sin(ang)
    else:
        c, s = cos_sin
    x = x.astype(np.float64)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def _rng(cfg: Config, *key: int) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, *key])


def _round(cfg: Config, x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return bf16_round(x) if cfg.dtype == "bf16" else x


def _draw_keys(cfg: Config, rng: np.random.Generator, n: int) -> np.ndarray:
    if cfg.key_dist == "student_t3":
        return rng.standard_t(3, size=(n, cfg.D)).astype(np.float32)
    return rng.standard_normal((n, cfg.D), dtype=np.float32)


def queries(cfg: Config, layer: int, lens: Optional[np.ndarray] = None) -> np.ndarray:
    """q_l [B, Hq, D] float32 (bf16-representable for bf16 configs)."""
    lens = cfg.lengths() if lens is None else lens
    q = np.empty((cfg.B, cfg.Hq, cfg.D), dtype=np.float32)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            v = _rng(cfg, layer, _Q, b, h).standard_normal(cfg.D, dtype=np.float32)
            if cfg.rope_base is not None:
                pos = np.array([max(int(lens[b]) - 1, 0)])
                v = rope_rotate(v[None, :], pos, cfg.rope_base)[0]
            q[b, h] = _round(cfg, v)
    return q


def salient_sets(cfg: Config, b: int, g: int, T_b: int) -> Tuple[np.ndarray, List[np.ndarray]]:
    """S_0 and the refined layers' S_l (l = 1..L) for one unit; sorted int64 arrays."""
    n = min(cfg.n_salient, T_b)
    if n == 0:
        return np.zeros(0, np.int64), [np.zeros(0, np.int64) for _ in range(cfg.n_refined)]
    rng = _rng(cfg, 0, _SAL, b, g)
    S0 = np.sort(rng.choice(T_b, size=n, replace=False).astype(np.int64))
    s0set = set(S0.tolist())
    layers = []
    for l in range(1, cfg.n_refined + 1):
        r = _rng(cfg, l, _SHIFT, b, g)
        n_shift = int(round(cfg.shift_frac * n))
        members = list(S0.tolist())
        which = r.choice(n, size=n_shift, replace=False) if n_shift else np.zeros(0, np.int64)
        taken = set(members)
        for i in which:
            s = members[i]
            for _ in range(1000):
                delta = int(r.integers(1, cfg.shift_max, endpoint=True))
                delta = delta if r.integers(0, 2) else -delta
                p = min(max(s + delta, 0), T_b - 1)
                if p not in taken and p not in s0set:
                    break
            else:
                continue
            taken.discard(s)
            taken.add(p)
            members[i] = p
        layers.append(np.sort(np.asarray(members, dtype=np.int64)))
    return S0, layers


def _unit_dir(q_group: np.ndarray) -> np.ndarray:
    s = q_group.astype(np.float64).sum(axis=0)
    nrm = np.linalg.norm(s)
    return s / nrm if nrm > 0 else s


def unit_tensors(cfg: Config, b: int, g: int, layer: int, q_layer: np.ndarray,
                 T_b: int, q_anchor: Optional[np.ndarray] = None,
                 want_v: Optional[bool] = None) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """K_l and V_l rows [T_max, D] (float32, bf16-representable for bf16 configs) of unit (b, g)."""
    D, G, T = cfg.D, cfg.G, cfg.T
    K = np.zeros((T, D), dtype=np.float32)
    raw = _draw_keys(cfg, _rng(cfg, layer, _K, b, g), T_b)
    if cfg.rope_base is not None and T_b > 0:
        cs = _rope_tables(T, D, cfg.rope_base)
        raw = rope_rotate(raw, np.arange(T_b), cfg.rope_base, (cs[0][:T_b], cs[1][:T_b]))
    K[:T_b] = raw
    S0, Sl = salient_sets(cfg, b, g, T_b)
    u = _unit_dir(q_layer[b, g * G:(g + 1) * G])
    if T_b > 0 and S0.size:
        plant = Sl[layer - 1] if layer >= 1 else S0
        K[plant] = (cfg.amp * math.sqrt(D) * u).astype(np.float32)
        if layer == 0:
            # rank-space locality: each shifted target sits at anchor rank r in [kappa, 3 kappa)
            targets = sorted(set().union(*[set(s.tolist()) for s in Sl]) - set(S0.tolist()))
            if targets:
                rr = _rng(cfg, 0, _RANK, b, g)
                sd = math.sqrt(3.0) if cfg.key_dist == "student_t3" else 1.0
                nd = NormalDist()
                for p in targets:
                    r = int(rr.integers(cfg.kappa, 3 * cfg.kappa))
                    frac = min(max((r + 0.5) / max(T_b, 1), 1e-9), 1 - 1e-9)
                    z = nd.inv_cdf(1.0 - frac) * sd
                    K[p] = (z * u).astype(np.float32)
    K = _round(cfg, K)
    if want_v is None:
        want_v = layer >= 1 or cfg.anchor_v
    V = None
    if want_v:
        V = np.zeros((T, D), dtype=np.float32)
        V[:T_b] = _rng(cfg, layer, _V, b, g).standard_normal((T_b, D), dtype=np.float32)
        V = _round(cfg, V)
    return K, V


@dataclass
class Workload:
    cfg: Config
    seq_lens: np.ndarray                 # [B] int32
    q: List[np.ndarray]                  # per layer [B,Hq,D] f32
    K: List[np.ndarray]                  # per layer [B,Hkv,T,D] f32
    V: List[Optional[np.ndarray]]        # per layer [B,Hkv,T,D] f32 or None (anchor)
    salient: Dict[Tuple[int, int], Tuple[np.ndarray, List[np.ndarray]]]

    @property
    def layers(self) -> int:
        return len(self.q)


def generate(cfg: Config, layers: Optional[Sequence[int]] = None, threads: int = 0) -> Workload:
    """Generate every layer (anchor + refined) of a config on the host.  Units are generated in
    a thread pool (each unit's draws are keyed independently, so the result does not depend on
    the thread count)."""
    lens = cfg.lengths()
    layers = list(range(cfg.n_refined + 1)) if layers is None else list(layers)
    threads = threads or min(16, os.cpu_count() or 1)
    qs, Ks, Vs = [], [], []
    for l in layers:
        q = queries(cfg, l, lens)
        K = np.zeros((cfg.B, cfg.Hkv, cfg.T, cfg.D), dtype=np.float32)
        want_v = l >= 1 or cfg.anchor_v
        V = np.zeros_like(K) if want_v else None

        def one(bg):
            b, g = bg
            k, v = unit_tensors(cfg, b, g, l, q, int(lens[b]))
            K[b, g] = k
            if V is not None:
                V[b, g] = v

        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, [(b, g) for b in range(cfg.B) for g in range(cfg.Hkv)]))
        qs.append(q)
        Ks.append(K)
        Vs.append(V)
    sal = {(b, g): salient_sets(cfg, b, g, int(lens[b])) for b in range(cfg.B) for g in range(cfg.Hkv)}
    return Workload(cfg=cfg, seq_lens=lens, q=qs, K=Ks, V=Vs, salient=sal)


def algorithmic_bytes(cfg: Config, seq_lens: Optional[np.ndarray] = None, key_bits: int = 8) -> Dict[str, float]:
    """Bytes the method must move per decode step (proposal + each refined layer), per unit:
    propose = T_b*D*key_bits/8 (compressed keys: int8, or 2-bit) + 4*T_b (scales) + G*D*e (query)
              + 4*kp (pool write)
    refine  = 4*kp (pool) + kp*D*e (gathered K rows) + kappa*D*e (gathered V rows)
              + 2*G*D*e (query in, output out) + 4*kappa (index write)
    where kp and kappa are capped by T_b as the method caps them."""
    e = 4 if cfg.dtype == "f32" else 2
    lens = cfg.lengths() if seq_lens is None else seq_lens
    prop = 0.0
    ref = 0.0
    for b in range(cfg.B):
        T_b = int(lens[b])
        kp_e = min(cfg.kp, T_b)
        ka_e = min(cfg.kappa, kp_e)
        for _ in range(cfg.Hkv):
            prop += T_b * cfg.D * key_bits // 8 + 4 * T_b + cfg.G * cfg.D * e + 4 * cfg.kp
            ref += 4 * cfg.kp + kp_e * cfg.D * e + ka_e * cfg.D * e + 2 * cfg.G * cfg.D * e + 4 * cfg.kappa
    return {"propose": prop, "refine_per_layer": ref, "step": prop + cfg.n_refined * ref}
