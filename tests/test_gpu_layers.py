"""The layer-wise slow step (sfi_slow_step_layers) against the fp64 oracle and against the
fused slow step (sfi_slow_step) called layer after layer.

Five layers share the ring slots, so every slot is reused; the Selector, the mask and (when
asked) the Reorg run on a second stream.  Every layer's out and lse are compared with the
oracle's dense step, its selection with the oracle's Selector run on the oracle's own logits
(sets equal up to near-ties at the Top-K boundary), its mask with the oracle's mask and its
compact segment with the oracle's Reorg of the selection; then every output must also equal
the sequential result bit for bit (the kernels are deterministic), and a fast step queued on
the primary stream right after the call must see the last layer's indices and compact segment
(the completion barrier) and match the oracle's fast step.
"""
import numpy as np
import pytest
import torch

from sparse_kv_attention_dense_amd import binding as B
from sparse_kv_attention_dense_amd import synth

from gpu_util import (DEV, assert_close_out, assert_close_rel, compare_index_sets, desc_for,
                      oracle_cache, round4, say, tolerances)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,n_slots,reorg,k_sel", [("gqa8_512k", 2, False, 1024),
                                                      ("ragged_paged_b16", 2, True, None),
                                                      ("gqa4_32k", 1, True, None)])
def test_layered_slow_step_matches_oracle_and_sequential(orc, name, n_slots, reorg, k_sel):
    base = synth.WORKLOADS[name]
    wl = base.scaled(7001, B=min(base.B, 3), len_lo=3000 if base.len_lo else None, k_sel=k_sel)
    n_layers = 5
    say(f"[layers] {wl.name} layers={n_layers} slots={n_slots} reorg={reorg}")
    lays = [synth.make_layer(wl, li, device=DEV) for li in range(n_layers)]
    lens = lays[0].len_at(0).to(DEV)
    max_len = lays[0].max_len_at(0)
    descs = [desc_for(lay, lens, max_len) for lay in lays]
    qs = [synth.make_query(wl, li, 0, device=DEV, u=lay.u) for li, lay in enumerate(lays)]
    stride = round4(max_len)
    istride = wl.n_sink + wl.k_sel
    frac = 0.25
    dense_ws = B.workspace(descs[0], idx_stride=istride, n_recent=wl.n_recent, device=DEV)

    def bufs():
        return dict(
            out=[torch.full((wl.B, wl.Hq, wl.d), float("nan"), device=DEV) for _ in lays],
            lse=[torch.full((wl.B, wl.Hq), float("nan"), device=DEV) for _ in lays],
            idx=[torch.full((wl.B, wl.Hkv, istride), -3, dtype=torch.int32, device=DEV) for _ in lays],
            n_idx=[torch.full((wl.B, wl.Hkv), -3, dtype=torch.int32, device=DEV) for _ in lays],
            mask=[torch.full((wl.B, wl.Hq), 7, dtype=torch.uint8, device=DEV) for _ in lays],
            logits=[torch.empty((wl.B, wl.Hq, stride), device=DEV) for _ in range(n_slots)],
            seg=[(torch.full((wl.B, wl.Hkv, istride, wl.d), float("nan"), dtype=wl.torch_dtype,
                             device=DEV),
                  torch.full((wl.B, wl.Hkv, istride, wl.d), float("nan"), dtype=wl.torch_dtype,
                             device=DEV),
                  torch.full((wl.B, wl.Hkv, istride), -9, dtype=torch.int32, device=DEV))
                 for _ in lays],
            sel_ws=[B.workspace(descs[0], idx_stride=istride, n_recent=wl.n_recent, device=DEV)
                    for _ in range(n_slots)])

    # sequential reference: the fused slow step, one layer after another
    ref = bufs()
    for l in range(n_layers):
        s = l % n_slots
        B.sfi_slow_step(descs[l], qs[l], ref["out"][l], ref["lse"][l], ref["logits"][s], stride,
                        wl.n_sink, wl.n_recent, wl.k_sel, ref["idx"][l], istride,
                        ref["n_idx"][l], frac, ref["mask"][l], ref["sel_ws"][s])
        if reorg:
            B.sfi_reorg(descs[l], ref["idx"][l], istride, ref["n_idx"][l], *ref["seg"][l])
    torch.cuda.synchronize()

    got = bufs()
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    events = [torch.cuda.Event() for _ in range(n_slots)]
    B.sfi_slow_step_layers(descs, qs, got["out"], got["lse"], got["logits"], stride,
                           got["sel_ws"], dense_ws, wl.n_sink, wl.n_recent, wl.k_sel, got["idx"],
                           istride, got["n_idx"], frac, got["mask"], stream, side, events,
                           torch.cuda.Event(), torch.cuda.Event(),
                           segments=got["seg"] if reorg else None)
    # queued on the primary stream right after: must see the last layer's indices and mask
    lens1 = lays[0].len_at(1).to(DEV)
    d1 = desc_for(lays[-1], lens1, lays[0].max_len_at(1))
    q1 = synth.make_query(wl, n_layers - 1, 1, device=DEV, u=lays[-1].u)
    fast_got = torch.empty((wl.B, wl.Hq, wl.d), device=DEV)
    B.sfi_sparse_decode(d1, q1, got["idx"][-1], istride, got["n_idx"][-1], wl.n_recent,
                        got["mask"][-1], fast_got, None, dense_ws)
    seg_got = torch.empty_like(fast_got)
    if reorg:
        B.sfi_sparse_decode_compact(d1, q1, *got["seg"][-1], istride, got["n_idx"][-1],
                                    wl.n_recent, got["mask"][-1], seg_got, None, dense_ws)
    torch.cuda.synchronize()
    fast_ref = torch.empty_like(fast_got)
    B.sfi_sparse_decode(d1, q1, ref["idx"][-1], istride, ref["n_idx"][-1], wl.n_recent,
                        ref["mask"][-1], fast_ref, None, dense_ws)
    torch.cuda.synchronize()

    # every layer against the oracle
    tol = tolerances(wl)
    lens_host = lays[0].len0_host
    swaps = 0
    for l in range(n_layers):
        cache = oracle_cache(orc, lays[l], lens_host)
        eo, el, ez = orc.dense(cache, qs[l])
        assert_close_out(got["out"][l].cpu().numpy(), eo, tol["out"], f"layer {l} out")
        assert_close_rel(got["lse"][l].cpu().numpy(), el, tol["rel"], f"layer {l} lse")
        eidx, en, f = orc.select(lens_host, wl.Hq, wl.Hkv, ez, wl.n_sink, wl.n_recent, wl.k_sel,
                                 istride, want_f=True)
        swaps += compare_index_sets(got["idx"][l], got["n_idx"][l], eidx, en, f, lens_host,
                                    wl.n_sink, wl.n_recent, wl.k_sel, exact=False)
        ehm = orc.sink_mask(ez[:, :, 0], el, frac)
        assert (got["mask"][l].cpu().numpy() == ehm).all(), f"mask differs at layer {l}"
        if reorg:
            ck, cv, cpos = orc.reorg(cache, got["idx"][l], got["n_idx"][l])
            gk, gv, gp = (x.cpu() for x in got["seg"][l])
            as_bits = (lambda t: t.view(torch.int16).numpy().view(np.uint16)) \
                if gk.dtype == torch.bfloat16 else (lambda t: t.numpy())
            assert (gp.numpy() == cpos).all(), f"segment positions differ at layer {l}"
            live = cpos >= 0
            assert (as_bits(gk)[live] == ck[live]).all(), f"segment keys differ at layer {l}"
            assert (as_bits(gv)[live] == cv[live]).all(), f"segment values differ at layer {l}"
        if l == n_layers - 1:
            lens_t = [n + 1 for n in lens_host]
            xo, _ = orc.sparse(oracle_cache(orc, lays[l], lens_t), q1, eidx, en, wl.n_recent, ehm)
            assert_close_out(fast_got.cpu().numpy(), xo, tol["out"], "fast step after the call")
    say(f"    oracle: every layer's out, lse, selection ({swaps} near-tie swaps), mask"
        f"{' and segment' if reorg else ''} agree")

    for key in ("out", "lse", "idx", "n_idx", "mask"):
        for l in range(n_layers):
            assert torch.equal(got[key][l], ref[key][l]), f"{key} differs at layer {l}"
    assert torch.equal(fast_got, fast_ref)
    if reorg:
        for l in range(n_layers):
            for a, b_ in zip(got["seg"][l], ref["seg"][l]):
                assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                                   b_.view(torch.int16) if b_.dtype == torch.bfloat16 else b_)
        assert torch.equal(seg_got, fast_ref)     # the compact segment of the last layer
    say(f"    {n_layers} layers identical to the sequential calls; fast step after the call too")
