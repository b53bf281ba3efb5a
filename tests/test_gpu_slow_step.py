"""sfi_slow_step (dense step with logits, Selector and mask in one call, the Selector's
normaliser over J kept by the dense kernels) against the fp64 oracle, and against the separate
calls sfi_dense_decode + sfi_select + sfi_sink_bypass_mask on the same inputs.

out, lse and logits come from the same dense kernels as sfi_dense_decode and must equal its
results bit for bit.  The selection is compared with the oracle's Selector run on the oracle's
own logits (sets equal up to near-ties at the Top-K boundary), and with sfi_select run on the
same GPU logits: the two normalisers over J differ in the last bits only, so the sets may
differ only at positions whose evidence (fp64, from the GPU logits) lies within 1e-5 of the
k-th largest."""
import numpy as np
import pytest
import torch

from sparse_kv_attention_dense_amd import binding as B
from sparse_kv_attention_dense_amd import synth

from gpu_util import (DEV, assert_close_out, assert_close_rel, assert_logits, compare_index_sets,
                      desc_for, gpu_dense, gpu_select, oracle_cache, round4, say, tolerances)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _slow(lay, q, t=0, max_len=None, n_sink=None, n_recent=None, k_sel=None, frac=None,
          ws=None, dense_done=None):
    wl = lay.wl
    n_sink = wl.n_sink if n_sink is None else n_sink
    n_recent = wl.n_recent if n_recent is None else n_recent
    k_sel = wl.k_sel if k_sel is None else k_sel
    frac = wl.mask_frac if frac is None else frac
    lens = lay.len_at(t).to(DEV)
    max_len = max_len or lay.max_len_at(t)
    desc = desc_for(lay, lens, max_len)
    stride = round4(max(max_len, 1))
    istride = n_sink + k_sel
    out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), device=DEV)
    lse = torch.full((wl.B, wl.Hq), float("nan"), device=DEV)
    logits = torch.full((wl.B, wl.Hq, stride), float("nan"), device=DEV)
    idx = torch.full((wl.B, wl.Hkv, max(istride, 1)), -7, dtype=torch.int32, device=DEV)
    n_idx = torch.full((wl.B, wl.Hkv), -7, dtype=torch.int32, device=DEV)
    mask = torch.full((wl.B, wl.Hq), 9, dtype=torch.uint8, device=DEV) if frac > 0 else None
    if ws is None:
        ws = torch.zeros(B.sfi_workspace_bytes(desc, B.SFI_OP_SLOW), dtype=torch.uint8,
                         device=DEV)
    B.sfi_slow_step(desc, q, out, lse, logits, stride, n_sink, n_recent, k_sel, idx,
                    max(istride, 1), n_idx, frac, mask, ws, dense_done=dense_done)
    torch.cuda.synchronize()
    return out, lse, logits, stride, idx, n_idx, mask


def _check_against_oracle(orc, lay, q, res, n_sink=None, n_recent=None, k_sel=None, frac=None):
    wl = lay.wl
    n_sink = wl.n_sink if n_sink is None else n_sink
    n_recent = wl.n_recent if n_recent is None else n_recent
    k_sel = wl.k_sel if k_sel is None else k_sel
    frac = wl.mask_frac if frac is None else frac
    out, lse, logits, stride, idx, n_idx, mask = res
    tol = tolerances(wl)
    eo, el, ez = orc.dense(oracle_cache(orc, lay, lay.len0_host), q)
    assert_close_out(out.cpu().numpy(), eo, tol["out"])
    assert_close_rel(lse.cpu().numpy(), el, tol["rel"], "lse")
    assert_logits(logits, ez, lay.len0_host, tol["rel"])
    eidx, en, f = orc.select(lay.len0_host, wl.Hq, wl.Hkv, ez, n_sink, n_recent, k_sel,
                             idx.shape[-1], want_f=True)
    swaps = compare_index_sets(idx, n_idx, eidx, en, f, lay.len0_host, n_sink, n_recent, k_sel,
                               exact=False)
    say(f"    selection against the oracle chain: {swaps} near-tie swaps")
    if mask is not None:
        ehm = orc.sink_mask(ez[:, :, 0], el, frac)
        assert (mask.cpu().numpy() == ehm).all()
    return ez


def _check_against_separate_calls(orc, lay, q, res, n_sink=None, n_recent=None, k_sel=None,
                                  max_len=None):
    wl = lay.wl
    n_sink = wl.n_sink if n_sink is None else n_sink
    n_recent = wl.n_recent if n_recent is None else n_recent
    k_sel = wl.k_sel if k_sel is None else k_sel
    out, lse, logits, stride, idx, n_idx, mask = res
    lens = lay.len_at(0).to(DEV)
    max_len = max_len or lay.max_len_at(0)
    desc = desc_for(lay, lens, max_len)
    ws = B.workspace(desc, idx_stride=idx.shape[-1], n_recent=n_recent, device=DEV)
    o2 = torch.full_like(out, float("nan"))
    l2 = torch.full_like(lse, float("nan"))
    z2 = torch.full_like(logits, float("nan"))
    B.sfi_dense_decode(desc, q, o2, l2, z2, stride, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    n = max(lay.len0_host)
    for b, nb in enumerate(lay.len0_host):
        assert torch.equal(logits[b, :, :nb], z2[b, :, :nb])
    i2, n2 = gpu_select(lens, max_len, wl, z2, stride, n_sink, n_recent, k_sel, idx.shape[-1],
                        ws=ws)
    _, _, f = orc.select(lay.len0_host, wl.Hq, wl.Hkv, z2[:, :, :max(n, 1)], n_sink, n_recent,
                         k_sel, idx.shape[-1], want_f=True)
    swaps = compare_index_sets(idx, n_idx, i2.cpu().numpy(), n2.cpu().numpy(), f,
                               lay.len0_host, n_sink, n_recent, k_sel, exact=False)
    say(f"    against sfi_dense_decode + sfi_select: out/lse/logits identical, "
        f"{swaps} near-tie swaps in the selection")


CASES = {
    "tiny_2k_f32": W["tiny_2k_f32"],
    "gqa4_32k": W["gqa4_32k"].scaled(9001),
    "sink_128k_b4": W["sink_128k_b4"].scaled(20001, B=2),
    "ragged_paged_b16": W["ragged_paged_b16"].scaled(9000, B=4, len_lo=3000),
    "gqa8_512k": W["gqa8_512k"].scaled(30001, k_sel=2048),
    # one KV head over 1.2M positions: 938 dense splits per head, so the merge runs 1024
    # threads and folds the splits' sums over J in several batches past the first 256
    "gqa8_512k_tp8": W["gqa8_512k_tp8"].scaled(1200003, k_sel=2048),
}


@pytest.mark.parametrize("name", list(CASES))
def test_slow_step_matches_oracle_and_separate_calls(orc, name):
    wl = CASES[name]
    say(f"[slow step] {wl.name} B={wl.B}")
    lay = synth.make_layer(wl, 0, device=DEV)
    q = synth.make_query(wl, 0, 0, device=DEV, u=lay.u)
    res = _slow(lay, q)
    _check_against_oracle(orc, lay, q, res)
    _check_against_separate_calls(orc, lay, q, res)


@pytest.mark.parametrize("path,n0,Bsz", [("unit", 6007, 2), ("chunked", 40000, 1)])
def test_slow_step_both_selector_paths(orc, path, n0, Bsz):
    """The one-workgroup Selector (a short context: one sequence of 6K) and the chunked one (one
    sequence of 40K, where the plan's estimate picks it) both take the normaliser from the dense
    step."""
    wl = W["gqa4_32k"].scaled(n0, B=Bsz)
    lay = synth.make_layer(wl, 1, device=DEV)
    q = synth.make_query(wl, 1, 0, device=DEV, u=lay.u)
    res = _slow(lay, q)
    _check_against_oracle(orc, lay, q, res)
    _check_against_separate_calls(orc, lay, q, res)


@pytest.mark.parametrize("G,d,dtype", [(1, 64, "bf16"), (16, 128, "bf16"), (8, 128, "f32"),
                                       (3, 64, "f32")])
def test_slow_step_head_shapes(orc, G, d, dtype):
    import dataclasses
    wl = dataclasses.replace(W["gqa4_32k"].scaled(5003, B=2, k_sel=700), Hq=2 * G, Hkv=2, d=d,
                             dtype=dtype, name=f"slow_G{G}_d{d}_{dtype}")
    lay = synth.make_layer(wl, 2, device=DEV)
    q = synth.make_query(wl, 2, 0, device=DEV, u=lay.u)
    res = _slow(lay, q)
    _check_against_oracle(orc, lay, q, res)
    _check_against_separate_calls(orc, lay, q, res)


@pytest.mark.parametrize("n_sink,n_recent,k_sel", [(0, 0, 500), (4, 256, 0), (4, 3000, 64),
                                                   (4, 5000, 64), (16, 100, 10000),
                                                   (0, 2049, 2048)])
def test_slow_step_edges_of_the_allowed_set(orc, n_sink, n_recent, k_sel):
    """No sinks or no recent window; k = 0; J shorter than k, empty for some sequences (every
    length here is at most 5003 + 1000), and J boundaries inside split and chunk tails."""
    wl = W["ragged_paged_b16"].scaled(5003, B=3, len_lo=4000)
    lay = synth.make_layer(wl, 3, device=DEV)
    q = synth.make_query(wl, 3, 0, device=DEV, u=lay.u)
    kw = dict(n_sink=n_sink, n_recent=n_recent, k_sel=k_sel)
    res = _slow(lay, q, **kw)
    _check_against_oracle(orc, lay, q, res, **kw)
    _check_against_separate_calls(orc, lay, q, res, **kw)


@pytest.mark.parametrize("case", range(8))
def test_slow_step_random_shapes(orc, case):
    """Seeded random slow steps (dense step, Selector and mask in one call): batch 1-3 with
    lengths 1-20000, 1-4 KV heads, groups of 1-8 query heads, d 64 or 128, bf16 or fp32, a
    contiguous or 16-position paged cache, 0-8 sinks, a recent window of 0-500, a budget of
    1-3000 and a mask over a quarter of the heads on odd cases; against the oracle chain and
    the separate calls."""
    import dataclasses
    rng = np.random.default_rng(4000 + case)
    Bn = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    paged = bool(rng.integers(0, 2))
    lens = [int(x) for x in rng.integers(1, 20001, size=Bn)]
    n_sink = int(rng.integers(0, 9))
    n_recent = int(rng.integers(0, 501))
    k_sel = int(rng.integers(1, 3001))
    wl = synth.Workload(f"slow_rand{case}", 9700 + case, Bn, Hkv * G, Hkv, d, dtype, max(lens),
                        n_sink, n_recent, k_sel, 2, paged=paged, block_size=16,
                        mask_frac=0.25 if case % 2 else 0.0)
    say(f"[slow random {case}] B={Bn} Hkv={Hkv} G={G} d={d} {dtype} paged={paged} lens={lens} "
        f"sink={n_sink} recent={n_recent} k={k_sel} mask={wl.mask_frac}")
    lay = synth.make_layer(wl, 0, device=DEV, lens=lens)
    q = synth.make_query(wl, 0, 0, device=DEV)
    res = _slow(lay, q)
    _check_against_oracle(orc, lay, q, res)
    _check_against_separate_calls(orc, lay, q, res)


def test_slow_step_full_size_128k(orc):
    """The 128K batch at full size in the benchmark's launch configuration: out, lse, logits
    identical to sfi_dense_decode; the selection against sfi_select on the same logits (near-ties
    only) and exact where the oracle's evidence margin is clear."""
    wl = W["sink_128k_b4"]
    lay = synth.make_layer(wl, 0, device=DEV)
    q = synth.make_query(wl, 0, 0, device=DEV, u=lay.u)
    ev = torch.cuda.Event()
    res = _slow(lay, q, dense_done=ev)
    assert ev.query()
    _check_against_separate_calls(orc, lay, q, res)
