"""Sparse fast step on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

from sparse_kv_attention_dense_amd import synth

from gpu_util import (DEV, assert_close_out, assert_close_rel, gpu_dense, gpu_sparse,
                      oracle_cache, say, tolerances)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _check(orc, lay, q, t, idx, n_idx, head_mask=None, n_recent=None):
    wl = lay.wl
    n_recent = wl.n_recent if n_recent is None else n_recent
    out, lse = gpu_sparse(lay, q, t, idx.to(DEV), n_idx.to(DEV),
                          None if head_mask is None else head_mask.to(DEV), n_recent=n_recent)
    lens = [n + t for n in lay.len0_host]
    eo, el = orc.sparse(oracle_cache(orc, lay, lens), q, idx, n_idx, n_recent, head_mask)
    tol = tolerances(wl)
    assert_close_out(out.cpu().numpy(), eo, tol["out"])
    assert_close_rel(lse.cpu().numpy(), el, tol["rel"], "lse")
    return out, lse


@pytest.mark.parametrize("kind", ["spans", "scattered"])
def test_sparse_ragged_paged(orc, kind):
    wl = W["ragged_paged_b16"].scaled(9000, B=4, len_lo=4000)
    say(f"[sparse] {wl.name} {kind}")
    lay = synth.make_layer(wl, 0, device=DEV)
    idx, n_idx = synth.synthetic_index_set(lay, kind, seed=21)
    for t in (1, 7):
        q = synth.make_query(wl, 0, t, device=DEV)
        _check(orc, lay, q, t, idx, n_idx)


@pytest.mark.parametrize("name", ["tiny_2k_f32", "gqa4_32k", "sink_128k_b4", "gqa8_512k"])
def test_sparse_contiguous(orc, name):
    base = W[name]
    wl = base if name == "tiny_2k_f32" else base.scaled(base.n_sink + base.k_sel + base.n_recent + 3001,
                                                         B=min(base.B, 2))
    say(f"[sparse] {wl.name}")
    lay = synth.make_layer(wl, 0, device=DEV)
    idx, n_idx = synth.synthetic_index_set(lay, "scattered", seed=22)
    q = synth.make_query(wl, 0, 3, device=DEV, u=lay.u)
    hm = None
    if wl.mask_frac > 0:
        g = torch.Generator().manual_seed(5)
        hm = (torch.rand((wl.B, wl.Hq), generator=g) < wl.mask_frac).to(torch.uint8)
    out, lse = _check(orc, lay, q, 3, idx, n_idx, head_mask=hm)
    if hm is not None:
        o = out.cpu()
        assert (o[hm.bool()] == 0).all()
        assert torch.isneginf(lse.cpu()[hm.bool()]).all()


def test_sparse_full_set_equals_dense(orc):
    """idx = every position before the recent window: the fast step is the dense step."""
    wl = W["gqa4_32k"].scaled(7001)
    lay = synth.make_layer(wl, 0, device=DEV)
    q = synth.make_query(wl, 0, 0, device=DEV)
    N = lay.len0_host[0]
    stride = N - wl.n_recent
    idx = torch.arange(stride, dtype=torch.int32).repeat(wl.B, wl.Hkv, 1).contiguous()
    n_idx = torch.full((wl.B, wl.Hkv), stride, dtype=torch.int32)
    so, sl = gpu_sparse(lay, q, 0, idx.to(DEV), n_idx.to(DEV))
    do, dl, _, _ = gpu_dense(lay, q, logits=False)
    err = (so - do).abs().max().item()
    say(f"    sparse(full) vs dense on GPU: {err:.3e}")
    assert err <= 1e-5
    assert (sl - dl).abs().max().item() <= 1e-5
    _check(orc, lay, q, 0, idx, n_idx)


def test_sparse_window_only_and_skipped_entries(orc):
    wl = synth.Workload("sp_edges", 8100, 3, 8, 2, 128, "bf16", 3000, 4, 100, 50, 2)
    lay = synth.make_layer(wl, 0, device=DEV, lens=[3000, 150, 90])
    q = synth.make_query(wl, 0, 1, device=DEV)
    # empty selection: window attention only
    idx = torch.zeros((3, 2, 60), dtype=torch.int32)
    _check(orc, lay, q, 1, idx, torch.zeros((3, 2), dtype=torch.int32))
    # ascending rows whose tail reaches into the recent window and past the length: those
    # entries are skipped (the recent run covers the window, positions >= len do not exist)
    rows, counts = [], []
    for N in (3001, 151, 91):
        r0 = max(0, N - wl.n_recent)
        row = sorted(set(range(0, min(20, r0))) | {r0, r0 + 1, N + 5, N + 9})
        counts.append(len(row))
        rows.append(row + [0] * (60 - len(row)))
    idx = torch.tensor(rows, dtype=torch.int32)[:, None, :].repeat(1, 2, 1).contiguous()
    n_idx = torch.tensor([[c, c] for c in counts], dtype=torch.int32)
    _check(orc, lay, q, 1, idx, n_idx)


def test_sparse_all_heads_masked_and_group_skip(orc):
    wl = W["gqa8_512k"].scaled(12000)
    lay = synth.make_layer(wl, 0, device=DEV)
    idx, n_idx = synth.synthetic_index_set(lay, "spans", seed=23)
    q = synth.make_query(wl, 0, 1, device=DEV, u=lay.u)
    hm = torch.zeros((1, wl.Hq), dtype=torch.uint8)
    hm[0, 8:16] = 1        # one whole KV group bypassed
    hm[0, 3] = 1           # and one head of another group
    out, lse = _check(orc, lay, q, 1, idx, n_idx, head_mask=hm)
    assert (out[0, 8:16] == 0).all() and (out[0, 3] == 0).all()


@pytest.mark.parametrize("name,samples", [("sink_128k_b4", [(0, 0), (3, 30)]),
                                          ("gqa8_512k", [(0, 5), (0, 60)])])
def test_sparse_full_size_sampled(orc, name, samples):
    wl = W[name]
    say(f"[sparse full] {wl.name}")
    lay = synth.make_layer(wl, 0, device=DEV)
    idx, n_idx = synth.synthetic_index_set(lay, "scattered", seed=24)
    t = wl.cycle - 1
    q = synth.make_query(wl, 0, t, device=DEV, u=lay.u)
    out, lse = gpu_sparse(lay, q, t, idx.to(DEV), n_idx.to(DEV))
    for b, i in samples:
        h = i // wl.G
        N = lay.len0_host[b] + t
        K1 = lay.k[b:b + 1, h:h + 1, :N].contiguous()
        V1 = lay.v[b:b + 1, h:h + 1, :N].contiguous()
        c = orc.Cache(K1, V1, torch.tensor([N], dtype=torch.int32), 1)
        eo, el = orc.sparse(c, q[b:b + 1, i:i + 1].contiguous(), idx[b:b + 1, h:h + 1].contiguous(),
                            n_idx[b:b + 1, h:h + 1].contiguous(), wl.n_recent)
        say(f"  sample b={b} i={i}")
        assert_close_out(out[b, i].cpu().numpy()[None, None], eo, 1e-2)
        assert_close_rel(lse[b, i:i + 1].cpu().numpy()[None], el, 1e-3, "lse")
    del lay
    torch.cuda.empty_cache()


def test_sparse_deterministic():
    wl = W["sink_128k_b4"].scaled(9000, B=2)
    lay = synth.make_layer(wl, 0, device=DEV)
    idx, n_idx = synth.synthetic_index_set(lay, "spans", seed=25)
    q = synth.make_query(wl, 0, 2, device=DEV, u=lay.u)
    a = gpu_sparse(lay, q, 2, idx.to(DEV), n_idx.to(DEV))
    b = gpu_sparse(lay, q, 2, idx.to(DEV), n_idx.to(DEV))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
