"""sfi_sparse_decode_noalloc (the fast step on the library's static scratch array, for callers
that cannot allocate) against sfi_sparse_decode on the same inputs, through the C ABI.

The two calls run the same kernels with the same launch plan; only the address of the partial
records differs, so the outputs must be identical bit for bit.  Two calls in a row on the
scratch array, the second with a smaller input, check that a call leaves nothing behind that
the next one depends on: the first is the 512K layer's fast step at full size (records of
1 MB), the second a 20K batch of two (records of half that), so the second call's records lie
inside what the first one wrote."""
import pytest
import torch

from sparse_kv_attention_dense_amd import binding as B
from sparse_kv_attention_dense_amd import synth

from gpu_util import DEV, desc_for, say

pytestmark = pytest.mark.gpu


def _selection(wl, lens, seed):
    """Sorted random selections of k_sel positions of J per (b, KV head), sinks first."""
    g = torch.Generator().manual_seed(seed)
    istride = wl.n_sink + wl.k_sel
    idx = torch.zeros((wl.B, wl.Hkv, istride), dtype=torch.int32)
    n_idx = torch.zeros((wl.B, wl.Hkv), dtype=torch.int32)
    for b, N in enumerate(lens):
        nJ = max(0, N - wl.n_recent - wl.n_sink)
        ns = min(wl.n_sink, N)
        for h in range(wl.Hkv):
            k = min(wl.k_sel, nJ)
            sel = torch.randperm(nJ, generator=g)[:k].sort().values.to(torch.int32) + wl.n_sink
            idx[b, h, :ns] = torch.arange(ns, dtype=torch.int32)
            idx[b, h, ns:ns + k] = sel
            n_idx[b, h] = ns + k
    return idx.to(DEV), n_idx.to(DEV), istride


def _case(wl, seed):
    lay = synth.make_layer(wl, 0, device=DEV)
    lens1 = [n + 1 for n in lay.len0_host]
    desc = desc_for(lay, lay.len_at(1).to(DEV), lay.max_len_at(1))
    q = synth.make_query(wl, 0, 1, device=DEV, u=lay.u)
    idx, n_idx, istride = _selection(wl, lens1, seed)
    mask = None
    if wl.mask_frac > 0:
        g = torch.Generator().manual_seed(seed + 1)
        mask = (torch.rand((wl.B, wl.Hq), generator=g) < wl.mask_frac).to(torch.uint8).to(DEV)
    return desc, q, idx, n_idx, istride, mask


def _compare(wl, case):
    desc, q, idx, n_idx, istride, mask = case
    need = B.sfi_workspace_bytes(desc, B.SFI_OP_SPARSE, istride, wl.n_recent)
    assert 0 < need <= B.SFI_NOALLOC_SCRATCH_BYTES
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    ref = torch.full((wl.B, wl.Hq, wl.d), float("nan"), device=DEV)
    ref_lse = torch.full((wl.B, wl.Hq), float("nan"), device=DEV)
    B.sfi_sparse_decode(desc, q, idx, istride, n_idx, wl.n_recent, mask, ref, ref_lse, ws)
    got = torch.full_like(ref, float("nan"))
    got_lse = torch.full_like(ref_lse, float("nan"))
    B.sfi_sparse_decode_noalloc(desc, q, idx, istride, n_idx, wl.n_recent, mask, got, got_lse)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    assert torch.equal(got, ref), f"out differs: max |diff| {float((got - ref).abs().max())}"
    assert torch.equal(got_lse, ref_lse)
    say(f"    {wl.name}: scratch output identical to the workspace call ({need} bytes of records)")
    return need


def test_noalloc_matches_workspace_call_twice_in_a_row():
    big = synth.WORKLOADS["gqa8_512k"]
    small = synth.WORKLOADS["sink_128k_b4"].scaled(20001, B=2, k_sel=1024)
    say(f"[noalloc] {big.name} then {small.name}")
    n_big = _compare(big, _case(big, 11))
    n_small = _compare(small, _case(small, 12))
    assert n_small < n_big
