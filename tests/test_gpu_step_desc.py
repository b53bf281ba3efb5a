"""Fast steps through the device step descriptor (sfi_step + sfi_sparse_decode_step).

Per-step state (cache pointers, lengths, block table, query, outputs, index set, mask,
compact segment, recent window) is written into one device struct before each step; the call
itself only carries shapes and capacity bounds.  Checked against the fp64 oracle's fast step
on the same index set, against the plain calls bit for bit, and replayed from one captured HIP
graph for every fast step of a cycle with only the descriptor rewritten between replays (each
replay bit-equal to the eager call of that step, with unrelated eager work in between)."""
import numpy as np
import pytest
import torch

from sparse_kv_attention_dense_amd import binding as B
from sparse_kv_attention_dense_amd import synth

from gpu_util import (DEV, assert_close_out, assert_close_rel, desc_for, oracle_cache, round4,
                      say, tolerances)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CASES = {
    "tiny_2k_f32": W["tiny_2k_f32"],
    "sink_128k_b4": W["sink_128k_b4"].scaled(20001, B=2),
    "ragged_paged_b16": W["ragged_paged_b16"].scaled(9000, B=3, len_lo=3000),
    "gqa8_512k": W["gqa8_512k"].scaled(30001, k_sel=2048),
}


def _slow_state(lay):
    """Slow step on the GPU: the index set (and mask) the fast steps reuse."""
    wl = lay.wl
    lens0 = lay.len_at(0).to(DEV)
    d0 = desc_for(lay, lens0, lay.max_len_at(0))
    stride = round4(lay.max_len_at(0))
    istride = wl.n_sink + wl.k_sel
    q0 = synth.make_query(wl, 0, 0, device=DEV, u=lay.u)
    out = torch.empty((wl.B, wl.Hq, wl.d), device=DEV)
    lse = torch.empty((wl.B, wl.Hq), device=DEV)
    logits = torch.empty((wl.B, wl.Hq, stride), device=DEV)
    idx = torch.empty((wl.B, wl.Hkv, istride), dtype=torch.int32, device=DEV)
    n_idx = torch.empty((wl.B, wl.Hkv), dtype=torch.int32, device=DEV)
    mask = torch.zeros((wl.B, wl.Hq), dtype=torch.uint8, device=DEV) if wl.mask_frac > 0 else None
    ws = B.workspace(desc_for(lay, lay.len_at(wl.cycle - 1).to(DEV), lay.max_len_at(wl.cycle - 1)),
                     idx_stride=istride, n_recent=wl.n_recent, device=DEV)
    B.sfi_slow_step(d0, q0, out, lse, logits, stride, wl.n_sink, wl.n_recent, wl.k_sel, idx,
                    istride, n_idx, wl.mask_frac, mask, ws)
    torch.cuda.synchronize()
    return idx, n_idx, mask, istride, ws


@pytest.mark.parametrize("name", list(CASES))
def test_step_descriptor_matches_oracle_and_plain_call(orc, name):
    wl = CASES[name]
    say(f"[step descriptor] {wl.name}")
    lay = synth.make_layer(wl, 0, device=DEV)
    idx, n_idx, mask, istride, ws = _slow_state(lay)
    tol = tolerances(wl)
    step = B.step_descriptor(DEV)
    shape = desc_for(lay, lay.len_at(0).to(DEV), lay.max_len_at(0))
    for t, n_recent in ((1, wl.n_recent), (2, wl.n_recent), (wl.cycle - 1, wl.n_recent),
                        (3, wl.n_recent // 2)):
        lens_t = lay.len_at(t).to(DEV)
        d_t = desc_for(lay, lens_t, lay.max_len_at(t))
        q_t = synth.make_query(wl, 0, t, device=DEV, u=lay.u)
        out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), device=DEV)
        lse = torch.full((wl.B, wl.Hq), float("nan"), device=DEV)
        B.write_step(step, d_t, q_t, idx, istride, n_idx, n_recent, mask, out, lse)
        B.sfi_sparse_decode_step(shape, step, istride, wl.n_recent, ws)
        torch.cuda.synchronize()
        xo, xl = orc.sparse(oracle_cache(orc, lay, [n + t for n in lay.len0_host]), q_t, idx,
                            n_idx, n_recent, mask)
        assert_close_out(out.cpu().numpy(), xo, tol["out"], f"t={t} n_recent={n_recent} out")
        assert_close_rel(lse.cpu().numpy(), xl, tol["rel"], f"t={t} lse")
        if n_recent == wl.n_recent:
            ref = torch.empty_like(out)
            ref_lse = torch.empty_like(lse)
            B.sfi_sparse_decode(d_t, q_t, idx, istride, n_idx, n_recent, mask, ref, ref_lse, ws)
            torch.cuda.synchronize()
            assert torch.equal(out, ref) and torch.equal(lse, ref_lse), f"step {t}"


@pytest.mark.parametrize("name,segment", [("sink_128k_b4", False), ("ragged_paged_b16", False),
                                          ("ragged_paged_b16", True), ("tiny_2k_f32", True)])
def test_step_descriptor_graph_serves_every_fast_step(name, segment):
    """One capture, replayed for steps 1 ... cycle - 1 with new lengths, query and output
    buffers each step (and, on the two-segment layout, the segment): only the descriptor is
    rewritten between replays."""
    wl = CASES[name]
    say(f"[step descriptor graph] {wl.name} segment={segment}")
    lay = synth.make_layer(wl, 0, device=DEV)
    idx, n_idx, mask, istride, ws = _slow_state(lay)
    seg = None
    if segment:
        d0 = desc_for(lay, lay.len_at(0).to(DEV), lay.max_len_at(0))
        ck = torch.empty((wl.B, wl.Hkv, istride, wl.d), dtype=wl.torch_dtype, device=DEV)
        cv = torch.empty_like(ck)
        cpos = torch.empty((wl.B, wl.Hkv, istride), dtype=torch.int32, device=DEV)
        B.sfi_reorg(d0, idx, istride, n_idx, ck, cv, cpos)
        seg = (ck, cv, cpos)
    shape = desc_for(lay, lay.len_at(0).to(DEV), lay.max_len_at(0))
    step = B.step_descriptor(DEV)
    # descriptor of step 1, then capture
    lens = [lay.len_at(t).to(DEV) for t in range(wl.cycle)]
    qs = [synth.make_query(wl, 0, t, device=DEV, u=lay.u) for t in range(wl.cycle)]
    outs = [torch.full((wl.B, wl.Hq, wl.d), float("nan"), device=DEV) for _ in range(wl.cycle)]
    lses = [torch.full((wl.B, wl.Hq), float("nan"), device=DEV) for _ in range(wl.cycle)]

    def write(t):
        d_t = desc_for(lay, lens[t], lay.max_len_at(t))
        if seg is None:
            B.write_step(step, d_t, qs[t], idx, istride, n_idx, wl.n_recent, mask, outs[t],
                         lses[t])
        else:
            B.write_step(step, d_t, qs[t], seg[2], istride, n_idx, wl.n_recent, mask, outs[t],
                         lses[t], segment=(seg[0], seg[1]))

    def call():
        B.sfi_sparse_decode_step(shape, step, istride, wl.n_recent, ws)

    write(1)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    ref = torch.empty_like(outs[0])
    ref_lse = torch.empty_like(lses[0])
    for t in range(1, wl.cycle):
        outs[t].fill_(float("nan"))
        write(t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # the eager call of this step (also unrelated eager work before the next replay)
        d_t = desc_for(lay, lens[t], lay.max_len_at(t))
        if seg is None:
            B.sfi_sparse_decode(d_t, qs[t], idx, istride, n_idx, wl.n_recent, mask, ref, ref_lse,
                                ws)
        else:
            B.sfi_sparse_decode_compact(d_t, qs[t], seg[0], seg[1], seg[2], istride, n_idx,
                                        wl.n_recent, mask, ref, ref_lse, ws)
        torch.cuda.synchronize()
        assert torch.equal(outs[t], ref) and torch.equal(lses[t], ref_lse), f"step {t}"
    say(f"    {wl.cycle - 1} replays of one capture, each identical to its step's eager call")
