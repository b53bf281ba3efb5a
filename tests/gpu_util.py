"""Helpers shared by the GPU parity tests: run the HIP library through its binding, run the
CPU oracle on the same input bytes, and compare with the documented tolerances.

Tolerances (fp32 outputs of the library against the fp64 oracle):
  * bf16 inputs: out max-abs <= 1e-2; logits |dz| <= 1e-3 * max(1, |z|); lse the same.
  * fp32 inputs: out max-abs <= 1e-5; logits and lse |d| <= 1e-5 * max(1, |x|).
  * index sets: identical on tie-free inputs; elsewhere the two sets may differ only at
    positions whose oracle evidence lies within 1e-5 (relative) of the k-th largest.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from sparse_kv_attention_dense_amd import binding as B
from sparse_kv_attention_dense_amd import synth

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def round4(n: int) -> int:
    return (n + 3) // 4 * 4


def tolerances(wl):
    if wl.dtype == "f32":
        return dict(out=1e-5, rel=1e-5)
    return dict(out=1e-2, rel=1e-3)


def desc_for(lay: synth.Layer, lens_dev, max_len: int) -> B.KVDesc:
    wl = lay.wl
    if wl.paged:
        return B.KVDesc(lay.k, lay.v, lens_dev, max_len, wl.Hq, block_table=lay.block_table,
                        block_size=wl.block_size)
    return B.KVDesc(lay.k, lay.v, lens_dev, max_len, wl.Hq)


def oracle_cache(orc, lay: synth.Layer, lens_host):
    wl = lay.wl
    kw = {}
    if wl.paged:
        kw = dict(block_table=lay.block_table, block_size=wl.block_size, max_blocks=lay.max_blocks)
    return orc.Cache(lay.k, lay.v, torch.tensor(lens_host, dtype=torch.int32), wl.Hq, **kw)


def workspace_for(desc: B.KVDesc, wl) -> torch.Tensor:
    return B.workspace(desc, idx_stride=wl.n_sink + wl.k_sel, n_recent=wl.n_recent, device=DEV)


def gpu_dense(lay: synth.Layer, q, t: int = 0, ws=None, logits: bool = True):
    wl = lay.wl
    lens = lay.len_at(t).to(DEV)
    max_len = lay.max_len_at(t)
    desc = desc_for(lay, lens, max_len)
    stride = round4(max(max_len, 1))
    out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), device=DEV)
    lse = torch.full((wl.B, wl.Hq), float("nan"), device=DEV)
    lg = torch.full((wl.B, wl.Hq, stride), float("nan"), device=DEV) if logits else None
    ws = workspace_for(desc, wl) if ws is None else ws
    B.sfi_dense_decode(desc, q, out, lse, lg, stride, ws)
    torch.cuda.synchronize()
    return out, lse, lg, stride


def gpu_select(lens_dev, max_len, wl, logits, stride, n_sink=None, n_recent=None, k_sel=None,
               idx_stride=None, ws=None):
    n_sink = wl.n_sink if n_sink is None else n_sink
    n_recent = wl.n_recent if n_recent is None else n_recent
    k_sel = wl.k_sel if k_sel is None else k_sel
    idx_stride = idx_stride or (n_sink + k_sel)
    Bsz = int(lens_dev.shape[0])
    desc = B.KVDesc.for_logits(lens_dev, max_len, wl.Hq, wl.Hkv, wl.d)
    idx = torch.full((Bsz, wl.Hkv, idx_stride), -7, dtype=torch.int32, device=DEV)
    n_idx = torch.full((Bsz, wl.Hkv), -7, dtype=torch.int32, device=DEV)
    if ws is None:
        ws = torch.zeros(B.sfi_workspace_bytes(desc, B.SFI_OP_SELECT), dtype=torch.uint8, device=DEV)
    B.sfi_select(desc, logits, stride, n_sink, n_recent, k_sel, idx, idx_stride, n_idx, ws)
    torch.cuda.synchronize()
    return idx, n_idx


def gpu_sparse(lay: synth.Layer, q, t: int, idx, n_idx, head_mask=None, ws=None, n_recent=None):
    wl = lay.wl
    n_recent = wl.n_recent if n_recent is None else n_recent
    lens = lay.len_at(t).to(DEV)
    desc = desc_for(lay, lens, lay.max_len_at(t))
    out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), device=DEV)
    lse = torch.full((wl.B, wl.Hq), float("nan"), device=DEV)
    if ws is None:
        ws = B.workspace(desc, idx_stride=idx.shape[-1], n_recent=n_recent, device=DEV)
    B.sfi_sparse_decode(desc, q, idx, idx.shape[-1], n_idx, n_recent, head_mask, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def assert_close_out(got, exp, tol, what="out"):
    got = np.asarray(got, np.float64)
    err = np.abs(got - exp)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    m = float(err.max()) if err.size else 0.0
    say(f"    {what}: max |err| = {m:.3e} (tol {tol:g})")
    assert m <= tol, f"{what}: max abs err {m} > {tol}"


def assert_close_rel(got, exp, rel, what):
    got = np.asarray(got, np.float64)
    fin = np.isfinite(exp)
    assert (np.isneginf(got) == np.isneginf(exp)).all(), f"{what}: -inf pattern differs"
    err = np.abs(got[fin] - exp[fin]) / np.maximum(1.0, np.abs(exp[fin]))
    m = float(err.max()) if err.size else 0.0
    say(f"    {what}: max rel err = {m:.3e} (tol {rel:g})")
    assert m <= rel, f"{what}: max rel err {m} > {rel}"


def assert_logits(got, exp, lens, rel):
    """got [B][Hq][stride] (device), exp [B][Hq][>=len] (oracle); rows compared over len."""
    g = got.cpu().numpy()
    worst = 0.0
    for b, n in enumerate(lens):
        d = np.abs(g[b, :, :n] - exp[b, :, :n]) / np.maximum(1.0, np.abs(exp[b, :, :n]))
        if d.size:
            worst = max(worst, float(d.max()))
    say(f"    logits: max rel err = {worst:.3e} (tol {rel:g})")
    assert worst <= rel


def compare_index_sets(idx_g, nidx_g, idx_o, nidx_o, f_o, lens, n_sink, n_recent, k_sel,
                       exact: bool, band: float = 1e-5):
    """Compare GPU and oracle selections per (b, h).  exact: sets must be identical.
    Otherwise differences are allowed only at positions whose oracle evidence is within
    `band` (relative) of the k_sel-th largest evidence.  Returns the number of such swaps."""
    ig, ng = idx_g.cpu().numpy(), nidx_g.cpu().numpy()
    swaps = 0
    for b in range(ig.shape[0]):
        N = int(lens[b])
        for h in range(ig.shape[1]):
            assert ng[b, h] == nidx_o[b, h], f"n_idx differs at ({b},{h}): {ng[b, h]} vs {nidx_o[b, h]}"
            g = ig[b, h, :ng[b, h]]
            o = idx_o[b, h, :nidx_o[b, h]]
            assert (np.diff(g) > 0).all(), f"GPU idx not strictly ascending at ({b},{h})"
            ns = min(n_sink, N)
            assert (g[:ns] == np.arange(ns)).all()
            if np.array_equal(g, o):
                continue
            assert not exact, f"index sets differ at ({b},{h})"
            J0, J1 = n_sink, N - n_recent
            assert ((g[ns:] >= J0) & (g[ns:] < J1)).all()
            fJ = f_o[b, h, J0:J1]
            kth = np.sort(fJ)[::-1][min(k_sel, len(fJ)) - 1]
            diff = np.setxor1d(g, o)
            near = np.abs(f_o[b, h, diff] - kth) <= band * kth
            assert near.all(), f"({b},{h}): sets differ away from the Top-K boundary"
            swaps += len(diff) // 2
    return swaps
