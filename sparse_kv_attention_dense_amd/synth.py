"""Seeded synthetic inputs for Slow-Fast decode attention.

This module only *draws* inputs: KV caches, queries, paged block tables,
planted logits and synthetic index sets.  It holds none of the attention,
selection or softmax arithmetic; both the HIP library's tests and the CPU
oracle read the tensors it returns.

Workload presets (one attention layer each):

* ``tiny_2k_f32``      batch 1, 4 query heads / 1 KV head, d=64, fp32, context 2048,
                       sink 4 + recent 64 + selected 128, cycle of 1 slow + 8 fast steps.
* ``gqa4_32k``         batch 1, 32/8 heads, d=128, bf16, context 32768,
                       sink 4 + recent 256 + selected 2048, cycle 16.
* ``sink_128k_b4``     batch 4, 32/8 heads, d=128, bf16, context 131072, token 0 is a
                       near-zero-value sink that draws about half the softmax mass,
                       sink 4 + recent 512 + selected 4096, cycle 16.
* ``ragged_paged_b16`` batch 16, 32/8 heads, d=128, bf16, lengths uniform in
                       [8192, 32768], paged KV in 16-token blocks with a shuffled block
                       table, selected 2048 as sentence-like spans or scattered positions,
                       sink 4 + recent 256, cycle 16.
* ``gqa8_512k``        batch 1, 64/8 heads, d=128, bf16, context 524288, sink recipe,
                       sink 4 + recent 1024 + selected 8192, cycle 32, bypass mask over
                       the 25% of query heads with the largest sink mass.

Sink recipe (SinkRouter, Sec. 3 "Insight": the BOS value has near-zero norm and the
BOS key sits apart from the semantic keys): a fixed random unit direction u per KV
head; every non-sink key has its u-component removed; key 0 becomes its
u-orthogonal part plus 8u; value 0 is rescaled to norm 1e-3; every query becomes its
u-orthogonal part plus s*u with s = (sqrt(d)/8) * (ln(N-1) + (d-1)/(2d)), which puts
about half of a head's softmax mass on token 0 at context N.

All values are drawn in fp32 from a ``torch.Generator`` seeded per preset, layer and
step, and rounded to bf16 with round-to-nearest-even where the preset is bf16.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed_base: int
    B: int
    Hq: int
    Hkv: int
    d: int
    dtype: str                 # "f32" or "bf16"
    n0: int                    # context length at the slow step (max when ragged)
    n_sink: int
    n_recent: int
    k_sel: int
    cycle: int                 # steps per slow-fast cycle: 1 slow + (cycle-1) fast
    sink: bool = False         # apply the sink recipe
    paged: bool = False
    block_size: int = 16
    len_lo: int = 0            # ragged lengths uniform in [len_lo, n0] when > 0
    mask_frac: float = 0.0     # bypass-mask fraction of query heads (0 = no mask)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def scaled(self, n0: int, B: Optional[int] = None, len_lo: Optional[int] = None,
               k_sel: Optional[int] = None, n_recent: Optional[int] = None,
               name_suffix: str = "small") -> "Workload":
        """Same structure at a smaller context (parity cases the oracle finishes fast)."""
        return dataclasses.replace(
            self, name=f"{self.name}_{name_suffix}", n0=n0,
            B=self.B if B is None else B,
            len_lo=(self.len_lo if len_lo is None else len_lo),
            k_sel=self.k_sel if k_sel is None else k_sel,
            n_recent=self.n_recent if n_recent is None else n_recent)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_2k_f32", 1000, 1, 4, 1, 64, "f32", 2048, 4, 64, 128, 9),
        Workload("gqa4_32k", 2000, 1, 32, 8, 128, "bf16", 32768, 4, 256, 2048, 16),
        Workload("sink_128k_b4", 3000, 4, 32, 8, 128, "bf16", 131072, 4, 512, 4096, 16,
                 sink=True),
        Workload("ragged_paged_b16", 4000, 16, 32, 8, 128, "bf16", 32768, 4, 256, 2048, 16,
                 paged=True, block_size=16, len_lo=8192),
        Workload("gqa8_512k", 5000, 1, 64, 8, 128, "bf16", 524288, 4, 1024, 8192, 32,
                 sink=True, mask_frac=0.25),
        # one GPU's share of gqa8_512k split by KV head over 8 GPUs (tensor-parallel
        # attention): one KV group of 8 query heads at the same context and budget
        Workload("gqa8_512k_tp8", 6000, 1, 8, 1, 128, "bf16", 524288, 4, 1024, 8192, 32,
                 sink=True, mask_frac=0.25),
    ]
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def sink_query_shift(d: int, n: int) -> float:
    """Query component along u that puts about half the softmax mass on token 0."""
    return (math.sqrt(d) / 8.0) * (math.log(max(n - 1, 1)) + (d - 1) / (2.0 * d))


@dataclasses.dataclass
class Layer:
    """One layer's KV cache, lengths and per-step queries for a workload."""
    wl: Workload
    k: torch.Tensor            # contiguous [B][Hkv][cap][d] or paged [n_blk][Hkv][bs][d]
    v: torch.Tensor
    len0: torch.Tensor         # int32 [B] lengths at the slow step (device)
    len0_host: list
    cap: int                   # rows per (b, h) for contiguous; max logical length
    block_table: Optional[torch.Tensor] = None   # int32 [B][max_blocks]
    max_blocks: int = 0
    u: Optional[torch.Tensor] = None             # fp32 [Hkv][d] sink direction

    def len_at(self, t: int) -> torch.Tensor:
        return self.len0 + t

    def max_len_at(self, t: int) -> int:
        return max(self.len0_host) + t


def _sink_dirs(wl: Workload, g: torch.Generator, device) -> torch.Tensor:
    u = torch.randn((wl.Hkv, wl.d), generator=g, device=device, dtype=torch.float32)
    return u / u.norm(dim=-1, keepdim=True)


def _fill_seq(wl: Workload, Kb: torch.Tensor, Vb: torch.Tensor, u: Optional[torch.Tensor]):
    """Apply the sink recipe in place to one sequence's fp32 [Hkv][n][d] K and V."""
    if u is None:
        return
    uu = u[:, None, :]                                        # [Hkv,1,d]
    Kb -= (Kb * uu).sum(-1, keepdim=True) * uu                # remove u from every key
    Kb[:, 0, :] += 8.0 * u                                    # key 0: orthogonal part + 8u
    v0 = Vb[:, 0, :]
    Vb[:, 0, :] = v0 * (1e-3 / v0.norm(dim=-1, keepdim=True))


def slow_step_lengths(wl: Workload) -> List[int]:
    """Sequence lengths at the slow step: n0 for every sequence, or for a ragged workload one
    draw per workload (every layer of a batch sees the same sequences)."""
    if wl.len_lo > 0:
        gl = _gen("cpu", wl.seed_base + 50)
        return torch.randint(wl.len_lo, wl.n0 + 1, (wl.B,), generator=gl).tolist()
    return [wl.n0] * wl.B


def make_layer(wl: Workload, layer: int = 0, device="cpu", lens=None) -> Layer:
    """Draw one layer's cache.  Capacity covers the whole cycle (n0 + cycle - 1 rows)."""
    seed = wl.seed_base + layer
    g = _gen(device, seed)
    dt = wl.torch_dtype
    # lengths at the slow step
    len_host = [int(x) for x in lens] if lens is not None else slow_step_lengths(wl)
    caps = [n + wl.cycle - 1 for n in len_host]
    cap = max(caps)
    u = _sink_dirs(wl, g, device) if wl.sink else None

    if not wl.paged:
        K = torch.empty((wl.B, wl.Hkv, cap, wl.d), dtype=dt, device=device)
        V = torch.empty_like(K)
        for b in range(wl.B):
            Kb = torch.randn((wl.Hkv, cap, wl.d), generator=g, device=device, dtype=torch.float32)
            Vb = torch.randn((wl.Hkv, cap, wl.d), generator=g, device=device, dtype=torch.float32)
            _fill_seq(wl, Kb, Vb, u)
            K[b] = Kb.to(dt)
            V[b] = Vb.to(dt)
            del Kb, Vb
        lay = Layer(wl, K, V, torch.tensor(len_host, dtype=torch.int32, device=device),
                    len_host, cap, u=u)
        return lay

    bs = wl.block_size
    nblk_seq = [(c + bs - 1) // bs for c in caps]
    max_blocks = max(nblk_seq)
    n_blk = sum(nblk_seq)
    gp = _gen("cpu", seed + 60)
    perm = torch.randperm(n_blk, generator=gp).to(torch.int32)
    bt = torch.zeros((wl.B, max_blocks), dtype=torch.int32)
    off = 0
    for b in range(wl.B):
        bt[b, :nblk_seq[b]] = perm[off:off + nblk_seq[b]]
        off += nblk_seq[b]
    K = torch.zeros((n_blk, wl.Hkv, bs, wl.d), dtype=dt, device=device)
    V = torch.zeros_like(K)
    bt_dev = bt.to(device)
    for b in range(wl.B):
        nb = nblk_seq[b]
        Kb = torch.randn((wl.Hkv, nb * bs, wl.d), generator=g, device=device, dtype=torch.float32)
        Vb = torch.randn((wl.Hkv, nb * bs, wl.d), generator=g, device=device, dtype=torch.float32)
        _fill_seq(wl, Kb, Vb, u)
        Kb[:, caps[b]:, :] = 0
        Vb[:, caps[b]:, :] = 0
        # [Hkv][nb][bs][d] -> [nb][Hkv][bs][d], scattered to the physical blocks
        Kp = Kb.view(wl.Hkv, nb, bs, wl.d).permute(1, 0, 2, 3).to(dt)
        Vp = Vb.view(wl.Hkv, nb, bs, wl.d).permute(1, 0, 2, 3).to(dt)
        phys = bt_dev[b, :nb].long()
        K[phys] = Kp
        V[phys] = Vp
        del Kb, Vb, Kp, Vp
    return Layer(wl, K, V, torch.tensor(len_host, dtype=torch.int32, device=device),
                 len_host, max(caps), block_table=bt_dev, max_blocks=max_blocks, u=u)


def steady_sink(layer: Layer, scale: float = 0.1):
    """Sink-heavy variant of the sink recipe (sink workloads): token 0's key keeps its 8u offset
    but its part orthogonal to u is scaled by `scale`, so its logit varies little from query to
    query (the stable first-token anchor that routing on a cached normaliser relies on).
    Rewrites the key rows of position 0 in place; returns what restore_sink puts back."""
    wl = layer.wl
    assert wl.sink and layer.u is not None
    saved = []
    for b in range(wl.B):
        rows = (layer.k[layer.block_table[b, 0].long(), :, 0, :] if wl.paged
                else layer.k[b, :, 0, :])                       # [Hkv][d]
        saved.append(rows.clone())
        k0 = rows.float()
        along = (k0 * layer.u).sum(-1, keepdim=True) * layer.u
        new = (scale * (k0 - along) + along).to(rows.dtype)
        if wl.paged:
            layer.k[layer.block_table[b, 0].long(), :, 0, :] = new
        else:
            layer.k[b, :, 0, :] = new
    return saved


def restore_sink(layer: Layer, saved):
    wl = layer.wl
    for b in range(wl.B):
        if wl.paged:
            layer.k[layer.block_table[b, 0].long(), :, 0, :] = saved[b]
        else:
            layer.k[b, :, 0, :] = saved[b]


def make_query(wl: Workload, layer: int, t: int, device="cpu", u=None, n_for_sink=None,
               sink_extra: float = 0.0):
    """Query for decode step t of a cycle ([B][Hq][d]).  sink_extra (sink workloads): raise
    token 0's logit by this many nats above the recipe's (ln 9 turns the recipe's even odds into
    about nine to one, a token-0 mass near 0.9)."""
    g = _gen(device, wl.seed_base + layer + 100 + t)
    q = torch.randn((wl.B, wl.Hq, wl.d), generator=g, device=device, dtype=torch.float32)
    if wl.sink:
        assert u is not None
        uq = u.repeat_interleave(wl.G, dim=0)[None]            # [1,Hq,d], head i -> KV head i//G
        s = sink_query_shift(wl.d, n_for_sink or wl.n0) + math.sqrt(wl.d) / 8.0 * sink_extra
        q = q - (q * uq).sum(-1, keepdim=True) * uq + s * uq
    return q.to(wl.torch_dtype)


def logical_kv(layer: Layer, b: int, h: int, n: int):
    """Rows [0, n) of sequence b, KV head h as fp32 [n][d] tensors (K, V)."""
    wl = layer.wl
    if not wl.paged:
        return layer.k[b, h, :n].float(), layer.v[b, h, :n].float()
    bs = wl.block_size
    nb = (n + bs - 1) // bs
    phys = layer.block_table[b, :nb].long()
    Kb = layer.k[phys, h].reshape(nb * bs, wl.d)[:n]
    Vb = layer.v[phys, h].reshape(nb * bs, wl.d)[:n]
    return Kb.float(), Vb.float()


# ---------------------------------------------------------------------------
# Synthetic selections (used where a test feeds the sparse step directly)
# ---------------------------------------------------------------------------

def span_selection(J_lo: int, J_hi: int, k: int, g: torch.Generator,
                   span_lo: int = 10, span_hi: int = 40) -> torch.Tensor:
    """k distinct positions in [J_lo, J_hi) laid out as sentence-like runs.

    Span lengths are uniform in [span_lo, span_hi]; the last span is trimmed so the
    total is exactly k; the free space is split into uniformly random gaps.
    """
    n = J_hi - J_lo
    if k >= n:
        return torch.arange(J_lo, J_hi, dtype=torch.int32)
    lens = []
    tot = 0
    while tot < k:
        L = int(torch.randint(span_lo, span_hi + 1, (1,), generator=g))
        L = min(L, k - tot)
        lens.append(L)
        tot += L
    free = n - k
    m = len(lens)
    # uniform composition of `free` into m+1 gaps via sorted cut points
    cuts = torch.sort(torch.randint(0, free + 1, (m,), generator=g)).values.tolist()
    gaps = [cuts[0]] + [cuts[i] - cuts[i - 1] for i in range(1, m)]
    out = []
    pos = J_lo
    for gp, L in zip(gaps, lens):
        pos += gp
        out.extend(range(pos, pos + L))
        pos += L
    return torch.tensor(out, dtype=torch.int32)


def scattered_selection(J_lo: int, J_hi: int, k: int, g: torch.Generator) -> torch.Tensor:
    n = J_hi - J_lo
    if k >= n:
        return torch.arange(J_lo, J_hi, dtype=torch.int32)
    pick = torch.randperm(n, generator=g)[:k]
    return (torch.sort(pick).values + J_lo).to(torch.int32)


def synthetic_index_set(layer: Layer, kind: str, seed: int, idx_stride: Optional[int] = None):
    """Ascending sink + selected positions per (b, h) with no selector involved.

    kind: "spans" or "scattered".  Returns (idx int32 [B][Hkv][stride], n_idx int32 [B][Hkv])
    on the CPU.
    """
    wl = layer.wl
    stride = idx_stride or (wl.n_sink + wl.k_sel)
    g = _gen("cpu", seed)
    idx = torch.zeros((wl.B, wl.Hkv, stride), dtype=torch.int32)
    n_idx = torch.zeros((wl.B, wl.Hkv), dtype=torch.int32)
    for b in range(wl.B):
        N = layer.len0_host[b]
        ns = min(wl.n_sink, N)
        J_lo, J_hi = wl.n_sink, N - wl.n_recent
        for h in range(wl.Hkv):
            if J_hi > J_lo:
                f = span_selection if kind == "spans" else scattered_selection
                sel = f(J_lo, J_hi, wl.k_sel, g)
            else:
                sel = torch.zeros(0, dtype=torch.int32)
            row = torch.cat([torch.arange(ns, dtype=torch.int32), sel])
            idx[b, h, :row.numel()] = row
            n_idx[b, h] = row.numel()
    return idx, n_idx


# ---------------------------------------------------------------------------
# Planted logits for the selector
# ---------------------------------------------------------------------------

def planted_logits(B: int, Hq: int, Hkv: int, lens, n_sink: int, n_recent: int,
                   stride: int, seed: int, alpha: float = 8.0, noise_sink: float = 0.0):
    """Logits whose group evidence ranks J by a known random permutation.

    For each (b, h) a permutation pi of J is drawn; every query head i of the group
    gets z[i, j] = -alpha * pi(j) / |J| + delta_i on J, with a per-head constant
    delta_i.  Positions outside J get arbitrary values (large ones when
    ``noise_sink`` > 0) because the selector must ignore them.  The expected top-k
    set is {j : pi(j) < k}.  Returns (logits fp32 [B][Hq][stride], ranks list).
    """
    G = Hq // Hkv
    g = _gen("cpu", seed)
    z = torch.randn((B, Hq, stride), generator=g, dtype=torch.float32)
    ranks = []
    for b in range(B):
        N = int(lens[b])
        J_lo, J_hi = n_sink, N - n_recent
        nJ = max(0, J_hi - J_lo)
        rb = []
        for h in range(Hkv):
            pi = torch.randperm(nJ, generator=g) if nJ > 0 else torch.zeros(0, dtype=torch.long)
            rb.append(pi)
            base = -alpha * pi.to(torch.float64) / max(nJ, 1)
            for gi in range(G):
                i = h * G + gi
                delta = float(torch.randn((1,), generator=g)) * 2.0
                if nJ > 0:
                    z[b, i, J_lo:J_hi] = (base + delta).to(torch.float32)
                if noise_sink > 0:
                    z[b, i, :min(n_sink, N)] = noise_sink
                    z[b, i, max(J_hi, n_sink):N] = noise_sink
                z[b, i, N:] = 0.0
        ranks.append(rb)
    return z, ranks
