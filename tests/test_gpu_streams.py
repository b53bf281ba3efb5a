"""Calls on two streams at once, each with its own workspace, against the same calls in turn.

The library keeps no state between calls and every call is asynchronous on the stream it is
given, so two slow-fast cycles queued on two streams (default priority) with separate
workspaces and outputs must give exactly the results of running them one after the other.
"""
import pytest
import torch

from sparse_kv_attention_dense_amd import binding as B
from sparse_kv_attention_dense_amd import synth

from gpu_util import DEV, desc_for, round4, say

pytestmark = pytest.mark.gpu


def _cycle(wl, lay, li, stream, bufs):
    """Slow step, Selector and two fast steps of layer li on `stream` into bufs."""
    with torch.cuda.stream(stream):
        lens = [lay.len_at(t).to(DEV) for t in range(3)]
        descs = [desc_for(lay, lens[t], lay.max_len_at(t)) for t in range(3)]
        qs = [synth.make_query(wl, li, t, device=DEV, u=lay.u) for t in range(3)]
        stride = bufs["logits"].shape[-1]
        istride = bufs["idx"].shape[-1]
        B.sfi_dense_decode(descs[0], qs[0], bufs["out"][0], bufs["lse"], bufs["logits"], stride,
                           bufs["ws"])
        B.sfi_select(descs[0], bufs["logits"], stride, wl.n_sink, wl.n_recent, wl.k_sel,
                     bufs["idx"], istride, bufs["n_idx"], bufs["ws"])
        for t in (1, 2):
            B.sfi_sparse_decode(descs[t], qs[t], bufs["idx"], istride, bufs["n_idx"], wl.n_recent,
                                None, bufs["out"][t], None, bufs["ws"])


def _bufs(wl, lay):
    stride = round4(lay.max_len_at(0))
    istride = wl.n_sink + wl.k_sel
    desc = desc_for(lay, lay.len_at(2).to(DEV), lay.max_len_at(2))
    return dict(out=[torch.full((wl.B, wl.Hq, wl.d), float("nan"), device=DEV) for _ in range(3)],
                lse=torch.full((wl.B, wl.Hq), float("nan"), device=DEV),
                logits=torch.full((wl.B, wl.Hq, stride), float("nan"), device=DEV),
                idx=torch.full((wl.B, wl.Hkv, istride), -1, dtype=torch.int32, device=DEV),
                n_idx=torch.full((wl.B, wl.Hkv), -1, dtype=torch.int32, device=DEV),
                ws=B.workspace(desc, idx_stride=istride, n_recent=wl.n_recent, device=DEV))


@pytest.mark.parametrize("name", ["sink_128k_b4", "ragged_paged_b16"])
def test_two_streams_match_sequential(name):
    base = synth.WORKLOADS[name]
    wl = base.scaled(20011, B=2, len_lo=9000 if base.len_lo else None)
    say(f"[streams] {wl.name}")
    lays = [synth.make_layer(wl, li, device=DEV) for li in range(2)]
    ref = [_bufs(wl, lay) for lay in lays]
    cur = torch.cuda.current_stream()
    for li, lay in enumerate(lays):
        _cycle(wl, lay, li, cur, ref[li])
    torch.cuda.synchronize()

    got = [_bufs(wl, lay) for lay in lays]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(cur)                                 # the buffers above are ready
    for li, lay in enumerate(lays):
        _cycle(wl, lay, li, streams[li], got[li])
    torch.cuda.synchronize()

    for li in range(2):
        for key in ("lse", "logits", "idx", "n_idx"):
            assert torch.equal(got[li][key].nan_to_num(7.0), ref[li][key].nan_to_num(7.0)), \
                f"layer {li}: {key} differs"
        for t in range(3):
            assert torch.equal(got[li]["out"][t], ref[li]["out"][t]), f"layer {li}: out[{t}] differs"
    say("    two concurrent cycles identical to the sequential ones")
