"""Sink-bypass mask on the GPU, and whole slow-fast cycles (dense -> select -> mask ->
fast steps) on the GPU against the same chain run by the oracle."""
import numpy as np
import pytest
import torch

from sparse_kv_attention_dense_amd import binding as B
from sparse_kv_attention_dense_amd import synth

from gpu_util import (DEV, assert_close_out, assert_close_rel, compare_index_sets, gpu_dense,
                      gpu_select, gpu_sparse, oracle_cache, round4, say, tolerances,
                      desc_for, workspace_for)

pytestmark = pytest.mark.gpu


def _gpu_mask(lens_dev, max_len, Hq, Hkv, logits, stride, lse, frac):
    desc = B.KVDesc.for_logits(lens_dev, max_len, Hq, Hkv)
    hm = torch.full(lse.shape, 9, dtype=torch.uint8, device=DEV)
    B.sfi_sink_bypass_mask(desc, logits, stride, lse, frac, hm)
    torch.cuda.synchronize()
    return hm


@pytest.mark.parametrize("frac", [0.0, 0.25, 0.3, 1.0])
def test_sink_mask_matches_oracle(orc, frac):
    g = torch.Generator().manual_seed(31)
    Bsz, Hq, Hkv, stride = 3, 64, 8, 16
    z = torch.randn((Bsz, Hq, stride), generator=g)
    lse = z[:, :, 0] + torch.rand((Bsz, Hq), generator=g) * 4
    # batch 2: four distinct token-0 masses, so the cut falls inside groups of exact ties
    z[2, :, 0] = 0.0
    lse[2] = torch.randint(1, 5, (Hq,), generator=g).float() / 2
    lens = torch.full((Bsz,), stride, dtype=torch.int32, device=DEV)
    hm = _gpu_mask(lens, stride, Hq, Hkv, z.to(DEV), stride, lse.to(DEV), frac)
    exp = orc.sink_mask(z[:, :, 0].double(), lse.double(), frac)
    assert (hm.cpu().numpy() == exp).all()
    assert int(hm.sum()) == Bsz * int(np.floor(frac * Hq))


W = synth.WORKLOADS
CYCLES = {
    "tiny_2k_f32": W["tiny_2k_f32"],
    "gqa4_32k": W["gqa4_32k"].scaled(6007),
    "sink_128k_b4": W["sink_128k_b4"].scaled(10001, B=2),
    "ragged_paged_b16": W["ragged_paged_b16"].scaled(7000, B=3, len_lo=3000),
    "gqa8_512k": W["gqa8_512k"].scaled(14001),
    "gqa8_512k_tp8": W["gqa8_512k_tp8"].scaled(15013),
}


@pytest.mark.parametrize("name", list(CYCLES))
def test_cycle_matches_oracle_chain(orc, name):
    """One slow step and the following fast steps, the GPU feeding itself and the oracle
    feeding itself; the selections must agree up to near-ties at the Top-K boundary and
    every output must agree to the output tolerance."""
    wl = CYCLES[name]
    say(f"[cycle] {wl.name} B={wl.B} cycle={wl.cycle}")
    lay = synth.make_layer(wl, 0, device=DEV)
    desc0 = desc_for(lay, lay.len_at(0).to(DEV), lay.max_len_at(0))
    ws = workspace_for(desc0, wl)
    tol = tolerances(wl)
    # slow step
    q0 = synth.make_query(wl, 0, 0, device=DEV, u=lay.u)
    out, lse, logits, stride = gpu_dense(lay, q0, 0, ws=ws)
    cache0 = oracle_cache(orc, lay, lay.len0_host)
    eo, el, ez = orc.dense(cache0, q0)
    assert_close_out(out.cpu().numpy(), eo, tol["out"])
    lens0 = lay.len_at(0).to(DEV)
    idx, n_idx = gpu_select(lens0, lay.max_len_at(0), wl, logits, stride, ws=ws)
    eidx, en, f = orc.select(lay.len0_host, wl.Hq, wl.Hkv, ez, wl.n_sink, wl.n_recent, wl.k_sel,
                             want_f=True)
    # GPU and oracle select from their own logits (fp32 vs fp64), so positions whose
    # evidence ties the k-th largest to within 1e-5 may swap; nothing else may differ
    swaps = compare_index_sets(idx, n_idx, eidx, en, f, lay.len0_host, wl.n_sink, wl.n_recent,
                               wl.k_sel, exact=False)
    say(f"    selection: {swaps} near-tie swaps at the Top-K boundary")
    hm, ehm = None, None
    if wl.mask_frac > 0:
        hm = _gpu_mask(lens0, lay.max_len_at(0), wl.Hq, wl.Hkv, logits, stride, lse, wl.mask_frac)
        ehm = orc.sink_mask(ez[:, :, 0], el, wl.mask_frac)
        assert (hm.cpu().numpy() == ehm).all()
    # fast steps reuse the selection while the recent window moves
    worst = 0.0
    for t in range(1, wl.cycle):
        qt = synth.make_query(wl, 0, t, device=DEV, u=lay.u)
        so, sl = gpu_sparse(lay, qt, t, idx, n_idx, head_mask=hm, ws=ws)
        lens_t = [n + t for n in lay.len0_host]
        xo, xl = orc.sparse(oracle_cache(orc, lay, lens_t), qt, eidx, en, wl.n_recent, ehm)
        err = float(np.abs(so.cpu().numpy() - xo).max())
        worst = max(worst, err)
        assert err <= tol["out"], f"fast step {t}: {err}"
        assert_close_rel(sl.cpu().numpy(), xl, tol["rel"], f"lse t={t}")
    say(f"    fast steps: worst max |err| = {worst:.3e}")
