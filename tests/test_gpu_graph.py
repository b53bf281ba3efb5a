"""The library's calls captured in a HIP graph (through torch.cuda.CUDAGraph) and replayed.

The calls queue kernels only (no memset, no host synchronisation, no allocation), so a
captured slow step (dense + Selector + mask) followed by fast steps must replay to exactly the
eager results.  Each replay is checked, with unrelated eager work on the same buffers in
between, so a node that only works on its first replay would show.
"""
import pytest
import torch

from sparse_kv_attention_dense_amd import binding as B
from sparse_kv_attention_dense_amd import synth

from gpu_util import DEV, desc_for, round4, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["gqa8_512k", "ragged_paged_b16"])
def test_graph_replay_matches_eager(name):
    base = synth.WORKLOADS[name]
    wl = base.scaled(9001, B=min(base.B, 3), len_lo=4000 if base.len_lo else None)
    say(f"[graph] {wl.name}")
    lay = synth.make_layer(wl, 0, device=DEV)
    T = 3                                          # slow step + 2 fast steps
    lens = [lay.len_at(t).to(DEV) for t in range(T)]
    descs = [desc_for(lay, lens[t], lay.max_len_at(t)) for t in range(T)]
    qs = [synth.make_query(wl, 0, t, device=DEV, u=lay.u) for t in range(T)]
    stride = round4(lay.max_len_at(0))
    istride = wl.n_sink + wl.k_sel
    ws = B.workspace(descs[-1], idx_stride=istride, n_recent=wl.n_recent, device=DEV)
    out = torch.empty((wl.B, wl.Hq, wl.d), device=DEV)
    lse = torch.empty((wl.B, wl.Hq), device=DEV)
    logits = torch.empty((wl.B, wl.Hq, stride), device=DEV)
    idx = torch.empty((wl.B, wl.Hkv, istride), dtype=torch.int32, device=DEV)
    n_idx = torch.empty((wl.B, wl.Hkv), dtype=torch.int32, device=DEV)
    mask = torch.zeros((wl.B, wl.Hq), dtype=torch.uint8, device=DEV)
    fast_out = [torch.empty_like(out) for _ in range(T)]
    frac = wl.mask_frac if wl.mask_frac > 0 else 0.25

    def cycle():
        B.sfi_dense_decode(descs[0], qs[0], out, lse, logits, stride, ws)
        B.sfi_select(descs[0], logits, stride, wl.n_sink, wl.n_recent, wl.k_sel, idx, istride,
                     n_idx, ws)
        B.sfi_sink_bypass_mask(descs[0], logits, stride, lse, frac, mask)
        fast_out[0].copy_(out)
        for t in range(1, T):
            B.sfi_sparse_decode(descs[t], qs[t], idx, istride, n_idx, wl.n_recent, mask,
                                fast_out[t], None, ws)

    def snapshot():
        torch.cuda.synchronize()
        return [x.clone() for x in (logits, lse, idx, n_idx, mask, *fast_out)]

    def scramble():
        for x in (logits, lse, out, *fast_out):
            x.fill_(float("nan"))
        idx.fill_(-5)
        n_idx.fill_(-5)
        mask.fill_(9)

    scramble()
    cycle()
    eager = snapshot()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cycle()                                    # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        cycle()
    for rep in range(3):
        # unrelated eager work on the same buffers between replays
        scramble()
        B.sfi_sparse_decode(descs[1], qs[2], idx.clamp(min=0), istride, n_idx.clamp(min=0),
                            wl.n_recent, None, out, None, ws)
        torch.cuda.synchronize()
        scramble()
        g.replay()
        got = snapshot()
        for k, (x, y) in enumerate(zip(got, eager)):
            assert torch.equal(x.nan_to_num(7.0), y.nan_to_num(7.0)), f"replay {rep}, buffer {k}"
        say(f"    replay {rep}: identical to eager")


def test_graph_fast_step_follows_device_state():
    """One captured fast step replayed for successive decode steps: the lengths (so the recent
    window) and the query are rewritten in device memory between replays, as a per-step
    descriptor is; the launch plan depends on max_len, idx_stride and n_recent only, so each
    replay equals, bit for bit, the eager call for that step."""
    base = synth.WORKLOADS["sink_128k_b4"]
    wl = base.scaled(9001, B=2)
    say(f"[graph] per-step device state {wl.name}")
    lay = synth.make_layer(wl, 0, device=DEV)
    T = wl.cycle
    max_len = lay.max_len_at(T - 1)                 # one bound for every step of the cycle
    lens_buf = lay.len_at(1).to(DEV).clone()
    q_buf = synth.make_query(wl, 0, 1, device=DEV, u=lay.u).clone()
    desc = desc_for(lay, lens_buf, max_len)
    idx, n_idx = synth.synthetic_index_set(lay, "spans", seed=41)
    idx, n_idx = idx.to(DEV), n_idx.to(DEV)
    istride = idx.shape[-1]
    ws = B.workspace(desc, idx_stride=istride, n_recent=wl.n_recent, device=DEV)
    out = torch.empty((wl.B, wl.Hq, wl.d), device=DEV)
    lse = torch.empty((wl.B, wl.Hq), device=DEV)

    def step():
        B.sfi_sparse_decode(desc, q_buf, idx, istride, n_idx, wl.n_recent, None, out, lse, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    ref_out = torch.empty_like(out)
    ref_lse = torch.empty_like(lse)
    for t in (1, 2, 7, T - 1):
        q_t = synth.make_query(wl, 0, t, device=DEV, u=lay.u)
        lens_t = lay.len_at(t).to(DEV)
        lens_buf.copy_(lens_t)
        q_buf.copy_(q_t)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        B.sfi_sparse_decode(desc_for(lay, lens_t, max_len), q_t, idx, istride, n_idx,
                            wl.n_recent, None, ref_out, ref_lse, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"step {t}"
        say(f"    step {t}: replay identical to the eager call")
