"""One decode step of the Prism hot path on the GPU: the proposal layer, then each refined layer
(Prism Attention page, Sec. 4 Overview: one anchor layer feeds the following shared layers;
Sec. 5.3 / Table 3 caption: g4 = one proposal layer and three refined layers).

Holds preallocated outputs and workspaces so that repeated steps allocate nothing; every step
runs through the C ABI of libprism.so on one stream.
"""
from dataclasses import dataclass
from typing import List, Optional

import torch

from . import binding as B


@dataclass
class LayerInputs:
    q: torch.Tensor                 # [B, Hq, D]
    K: torch.Tensor                 # [B, Hkv, T_max, D]
    V: Optional[torch.Tensor]       # [B, Hkv, T_max, D] (None for the anchor unless it attends)


class PrismStep:
    """Proposal on layer 0 (compressed keys Kq/scales: int8 codes, or with key_bits=2 the packed
    INT2 codes of quantize_keys_int2), then refine_attend on layers 1..L.

    With `anchor` (layer 0's exact K and V) the step also runs the anchor layer's own attention:
    refine_attend on layer 0 with the pool it just proposed, right after the proposal.  The pages
    give the anchor layer only the proposing role (Prism Attention page, Sec. 4 Overview), so the
    default step leaves it out; this variant is the anchor as a full attention layer of its group."""

    def __init__(self, q0: torch.Tensor, Kq: torch.Tensor, scales: torch.Tensor, refined: List[LayerInputs],
                 kp: int, kappa: int, agg: int = B.AGG_SUM, seq_lens: Optional[torch.Tensor] = None,
                 want_lse: bool = True, stream=None, ws_propose: Optional[torch.Tensor] = None,
                 ws_refine: Optional[torch.Tensor] = None, key_bits: int = 8,
                 anchor: Optional[LayerInputs] = None):
        if key_bits not in (8, 2):
            raise ValueError("key_bits must be 8 or 2")
        if anchor is not None and (anchor.V is None or anchor.q is not q0):
            raise ValueError("anchor attention needs layer 0's V and the proposal's own query")
        self.anchor = anchor
        self.key_bits = key_bits
        self.q0, self.Kq, self.scales = q0, Kq, scales
        self.refined = refined
        self.kp, self.kappa, self.agg = kp, kappa, agg
        self.seq_lens = seq_lens
        self.stream = stream
        dev = q0.device
        shape = B.make_shape(q0, Kq, seq_lens, k_cols_per_dim=4 if key_bits == 2 else 1)
        Bn, Hkv = shape.B, shape.Hkv
        self.pool = torch.empty((Bn, Hkv, kp), dtype=torch.int32, device=dev)
        # workspaces may be shared by steps that run one after another on the same stream
        self.ws_p = ws_propose if ws_propose is not None else B.new_workspace(
            B.OP_PROPOSE, shape, kp, 0, device=dev, stream=stream)
        self.ws_r = ws_refine
        first = refined[0] if refined else anchor
        if self.ws_r is None and first is not None:
            self.ws_r = B.new_workspace(B.OP_REFINE, B.make_shape(first.q, first.K, seq_lens), kp, kappa,
                                        device=dev, stream=stream)
        self.out = [torch.empty_like(L.q) for L in refined]
        self.idx = [torch.empty((Bn, Hkv, kappa), dtype=torch.int32, device=dev) for _ in refined]
        self.lse = [torch.empty((Bn, L.q.shape[1]), dtype=torch.float32, device=dev) if want_lse else None
                    for L in refined]
        if anchor is not None:
            self.out_anchor = torch.empty_like(anchor.q)
            self.idx_anchor = torch.empty((Bn, Hkv, kappa), dtype=torch.int32, device=dev)
            self.lse_anchor = torch.empty((Bn, anchor.q.shape[1]), dtype=torch.float32, device=dev) \
                if want_lse else None

    def propose(self):
        fn = B.propose_int2 if self.key_bits == 2 else B.propose
        return fn(self.q0, self.Kq, self.scales, self.kp, self.agg, seq_lens=self.seq_lens, pool=self.pool,
                  ws=self.ws_p, stream=self.stream)

    def refine(self, i: int):
        L = self.refined[i]
        return B.refine_attend(L.q, L.K, L.V, self.pool, self.kappa, self.agg, seq_lens=self.seq_lens,
                               out=self.out[i], idx=self.idx[i], lse=self.lse[i], want_lse=self.lse[i] is not None,
                               ws=self.ws_r, stream=self.stream)

    def attend_anchor(self):
        A = self.anchor
        return B.refine_attend(A.q, A.K, A.V, self.pool, self.kappa, self.agg, seq_lens=self.seq_lens,
                               out=self.out_anchor, idx=self.idx_anchor, lse=self.lse_anchor,
                               want_lse=self.lse_anchor is not None, ws=self.ws_r, stream=self.stream)

    def __call__(self):
        self.propose()
        if self.anchor is not None:
            self.attend_anchor()
        for i in range(len(self.refined)):
            self.refine(i)
        return self.pool, self.idx, self.out, self.lse

    def capture(self):
        """Record one whole step (proposal + every refined layer) into a HIP graph and return it.

        Nothing is allocated and no memset is issued while capturing, so replays are valid;
        each replay recomputes the step from the current contents of the input buffers."""
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self()
        self.graph = graph
        return graph
