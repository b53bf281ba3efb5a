"""Sparse fast step on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

from sparse_kv_attention_dense_amd import binding as B
from sparse_kv_attention_dense_amd import synth

from gpu_util import (DEV, assert_close_out, assert_close_rel, desc_for, gpu_dense, gpu_sparse,
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


@pytest.mark.parametrize("dtype,d,G,block", [("bf16", 64, 1, 0), ("bf16", 128, 16, 64),
                                             ("f32", 128, 2, 0), ("f32", 64, 8, 1),
                                             ("bf16", 128, 3, 16), ("bf16", 64, 7, 0)])
def test_sparse_head_shapes(orc, dtype, d, G, block):
    """Group sizes 1 to 16, d 64 and 128, fp32 and bf16, contiguous and paged caches with
    pages of 1, 16 and 64 positions; two steps of the moving recent window."""
    wl = synth.Workload(f"sparse_shape_{dtype}_{d}_{G}_{block}", 7400 + d + G + block, 2, 2 * G,
                        2, d, dtype, 1500, 4, 64, 128, 4, paged=block > 0,
                        block_size=max(block, 1))
    say(f"[sparse] {wl.name}")
    lay = synth.make_layer(wl, 0, device=DEV, lens=[1500, 777])
    idx, n_idx = synth.synthetic_index_set(lay, "spans", seed=31)
    for t in (1, 3):
        q = synth.make_query(wl, 0, t, device=DEV)
        _check(orc, lay, q, t, idx, n_idx)


@pytest.mark.parametrize("lens", [[5000, 3100], [3073, 40]])
def test_sparse_paged_long_block_table(orc, lens):
    """A block table longer than the 3072 entries a fast-step workgroup stages in LDS (pages of
    one position): the rows are then looked up in the table directly."""
    wl = synth.Workload("sparse_long_bt", 7700, 2, 8, 2, 128, "bf16", max(lens), 4, 64, 300, 2,
                        paged=True, block_size=1)
    say(f"[sparse] {wl.name} lens={lens}")
    lay = synth.make_layer(wl, 0, device=DEV, lens=lens)
    assert lay.max_blocks > 3072
    idx, n_idx = synth.synthetic_index_set(lay, "scattered", seed=33)
    q = synth.make_query(wl, 0, 1, device=DEV)
    _check(orc, lay, q, 1, idx, n_idx)


def test_sparse_largest_split(orc):
    """An index set long enough that each fast-step workgroup holds the largest split its row
    table allows (4096 slots): 1,049,068 slots for the one (sequence, KV head) unit, 257
    workgroups."""
    n = 1_050_000
    wl = synth.Workload("sparse_largest_split", 7600, 1, 2, 1, 64, "bf16", n, 4, 64, 1_049_000, 2)
    say(f"[sparse] {wl.name}")
    lay = synth.make_layer(wl, 0, device=DEV)
    idx, n_idx = synth.synthetic_index_set(lay, "scattered", seed=32)
    assert int(n_idx[0, 0]) + wl.n_recent > 256 * 4096
    q = synth.make_query(wl, 0, 1, device=DEV)
    _check(orc, lay, q, 1, idx, n_idx)


@pytest.mark.parametrize("case", range(12))
def test_sparse_random_shapes(orc, case):
    """Seeded random fast steps against the oracle: batch 1-4, 1-4 KV heads, groups of 1-16
    query heads, d 64 or 128, bf16 or fp32, a contiguous cache or pages of 1, 16 or 64
    positions, lengths 1-12000, 0-8 sinks, a recent window of 0-300, a budget of 1-3000 (often
    past the allowed set of the short sequences), span or scattered selections, a step 0-4
    tokens into the cycle, and on every third case a random head mask."""
    rng = np.random.default_rng(2000 + case)
    Bn = int(rng.integers(1, 5))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    block = int(rng.choice([0, 1, 16, 64]))
    lens = [int(x) for x in rng.integers(1, 12001, size=Bn)]
    n_sink = int(rng.integers(0, 9))
    n_recent = int(rng.integers(0, 301))
    k_sel = int(rng.integers(1, 3001))
    cycle = 5
    wl = synth.Workload(f"sp_rand{case}", 9000 + case, Bn, Hkv * G, Hkv, d, dtype, max(lens),
                        n_sink, n_recent, k_sel, cycle, paged=block > 0,
                        block_size=max(block, 1))
    kind = "spans" if case % 2 else "scattered"
    t = int(rng.integers(0, cycle))
    say(f"[sparse random {case}] B={Bn} Hkv={Hkv} G={G} d={d} {dtype} block={block} "
        f"lens={lens} sink={n_sink} recent={n_recent} k={k_sel} {kind} t={t}")
    lay = synth.make_layer(wl, 0, device=DEV, lens=lens)
    idx, n_idx = synth.synthetic_index_set(lay, kind, seed=40 + case)
    hm = None
    if case % 3 == 0:
        g = torch.Generator().manual_seed(60 + case)
        hm = (torch.rand((Bn, Hkv * G), generator=g) < 0.3).to(torch.uint8)
    q = synth.make_query(wl, 0, t, device=DEV)
    _check(orc, lay, q, t, idx, n_idx, head_mask=hm)


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


def test_sparse_without_recent_window(orc):
    """n_recent = 0: only the index set is attended; a unit with an empty index set attends to
    nothing (zero output, lse = -inf)."""
    wl = synth.Workload("sp_no_recent", 8200, 3, 8, 2, 128, "bf16", 3000, 4, 0, 300, 3)
    lay = synth.make_layer(wl, 0, device=DEV, lens=[3000, 700, 5])
    idx, n_idx = synth.synthetic_index_set(lay, "scattered", seed=25)
    n_idx[1, 1] = 0
    for t in (0, 2):
        q = synth.make_query(wl, 0, t, device=DEV)
        out, lse = _check(orc, lay, q, t, idx, n_idx, n_recent=0)
        assert (out[1, 4:8] == 0).all() and torch.isneginf(lse[1, 4:8]).all()


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
                                          ("gqa8_512k", [(0, 5), (0, 60)]),
                                          ("ragged_paged_b16", [(2, 3), (11, 28)]),
                                          ("gqa4_32k", [(0, 30)])])
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
        Kf, Vf = synth.logical_kv(lay, b, h, N)        # gathers through the block table when paged
        K1 = Kf.to(wl.torch_dtype)[None, None].contiguous()
        V1 = Vf.to(wl.torch_dtype)[None, None].contiguous()
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


def _routed_gpu(lay, q, t, idx, n_idx, route_lse, gamma, head_mask=None):
    wl = lay.wl
    lens = lay.len_at(t).to(DEV)
    desc = desc_for(lay, lens, lay.max_len_at(t))
    out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), device=DEV)
    lse = torch.full((wl.B, wl.Hq), float("nan"), device=DEV)
    routed = torch.full((wl.B, wl.Hkv), 9, dtype=torch.uint8, device=DEV)
    ws = B.workspace(desc, idx_stride=idx.shape[-1], n_recent=wl.n_recent, device=DEV)
    B.sfi_sparse_decode_routed(desc, q, idx.to(DEV), idx.shape[-1], n_idx.to(DEV), wl.n_recent,
                               None if head_mask is None else head_mask.to(DEV),
                               route_lse.to(DEV).float(), gamma, routed, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse, routed


@pytest.mark.parametrize("name", ["sink_128k_b4", "gqa8_512k", "ragged_paged_b16", "tiny_2k_f32"])
def test_sparse_routed_planted_decisions(orc, name):
    """Normalisers set head by head so the estimated token-0 mass is 0.9 or 0.3: every decision
    is far from the threshold and must match the oracle; outputs within tolerance."""
    base = W[name]
    wl = base if name == "tiny_2k_f32" else base.scaled(9001, B=min(base.B, 2),
                                                         len_lo=4000 if base.len_lo else None)
    _routed_planted(orc, wl)


@pytest.mark.parametrize("dtype,d,G,block", [("bf16", 128, 16, 0), ("f32", 64, 16, 16),
                                             ("bf16", 64, 1, 1)])
def test_sparse_routed_head_shapes(orc, dtype, d, G, block):
    """Routing with every thread of the prologue busy (16 heads x 16 lanes at d = 128), fp32 at
    d = 64 on a paged cache, and single-head groups on one-position pages."""
    wl = synth.Workload(f"routed_{dtype}_{d}_{G}_{block}", 7800 + d + G + block, 2, 2 * G, 2, d,
                        dtype, 3000, 4, 64, 300, 3, paged=block > 0, block_size=max(block, 1))
    _routed_planted(orc, wl)


def _routed_planted(orc, wl):
    say(f"[sparse routed planted] {wl.name}")
    lay = synth.make_layer(wl, 0, device=DEV)
    t = 2
    q = synth.make_query(wl, 0, t, device=DEV, u=lay.u)
    idx, n_idx = synth.synthetic_index_set(lay, "spans", seed=31)
    lens = [n + t for n in lay.len0_host]
    c = oracle_cache(orc, lay, lens)
    _, _, z = orc.dense(c, q)
    g = torch.Generator().manual_seed(7)
    # whole groups at 0.9 half of the time, otherwise a random mix of 0.9 and 0.3
    grp = (torch.rand((wl.B, wl.Hkv), generator=g) < 0.5).repeat_interleave(wl.G, dim=1)
    mix = torch.rand((wl.B, wl.Hq), generator=g) < 0.5
    target = torch.where(grp | mix, 0.9, 0.3).double()
    route_lse = torch.tensor(z[:, :, 0]) - torch.log(target)
    out, lse, routed = _routed_gpu(lay, q, t, idx, n_idx, route_lse, 0.65)
    eo, el, er, margin = orc.sparse_routed(c, q, idx, n_idx, wl.n_recent, route_lse, 0.65)
    assert (np.abs(margin) > 0.3).all()
    assert (routed.cpu().numpy() == er).all(), "routing decisions differ"
    say(f"    groups routed: {int(er.sum())} of {er.size}")
    tol = tolerances(wl)
    assert_close_out(out.cpu().numpy(), eo, tol["out"])
    assert_close_rel(lse.cpu().numpy(), el, tol["rel"], "lse")


def test_sparse_routed_with_slow_step_lse(orc):
    """The intended use: the slow step's lse as the cached normaliser and gamma = 0.65 on the
    sink-dominated workload.  Decisions must agree wherever rounding cannot flip them; outputs
    are checked against the oracle given the GPU's decisions."""
    wl = W["sink_128k_b4"].scaled(12001, B=2)
    lay = synth.make_layer(wl, 0, device=DEV)
    q0 = synth.make_query(wl, 0, 0, device=DEV, u=lay.u)
    _, lse0, _, _ = gpu_dense(lay, q0, 0, logits=False)
    t = 3
    q = synth.make_query(wl, 0, t, device=DEV, u=lay.u)
    idx, n_idx = synth.synthetic_index_set(lay, "scattered", seed=32)
    out, lse, routed = _routed_gpu(lay, q, t, idx, n_idx, lse0.cpu().double(), 0.65)
    lens = [n + t for n in lay.len0_host]
    c = oracle_cache(orc, lay, lens)
    _, _, er, margin = orc.sparse_routed(c, q, idx, n_idx, wl.n_recent, lse0.cpu().double(), 0.65)
    rg = routed.cpu().numpy()
    clear = np.abs(margin) > 1e-3
    assert (rg[clear] == er[clear]).all()
    say(f"    groups routed: {int(rg.sum())} of {rg.size}; near-threshold: {int((~clear).sum())}")
    hm = torch.tensor(rg).repeat_interleave(wl.G, dim=1).to(torch.uint8)
    eo, el = orc.sparse(c, q, idx, n_idx, wl.n_recent, hm)
    assert_close_out(out.cpu().numpy(), eo, 1e-2)
    assert_close_rel(lse.cpu().numpy(), el, 1e-3, "lse")


@pytest.mark.parametrize("name", ["sink_128k_b4", "gqa8_512k"])
def test_sparse_routed_sink_heavy_operating_point(orc, name):
    """The sink recipe with token 0's key steadied (its part orthogonal to the sink direction
    scaled by 0.1, so its logit varies little between queries) and its logit raised by ln 9
    (token-0 mass near 0.9): most KV groups reach gamma = 0.65 with the slow step's lse as
    normaliser, so the routed step skips their rows.  Decisions agree with the oracle's
    wherever rounding cannot flip them, outputs agree with the oracle given the GPU's decisions,
    and most groups are bypassed."""
    base = W[name]
    wl = base.scaled(16001, B=min(base.B, 2), k_sel=1024)
    lay = synth.make_layer(wl, 0, device=DEV)
    synth.steady_sink(lay, 0.1)
    extra = float(np.log(9.0))
    q0 = synth.make_query(wl, 0, 0, device=DEV, u=lay.u, sink_extra=extra)
    _, lse0, _, _ = gpu_dense(lay, q0, 0, logits=False)
    t = 5
    q = synth.make_query(wl, 0, t, device=DEV, u=lay.u, sink_extra=extra)
    idx, n_idx = synth.synthetic_index_set(lay, "scattered", seed=34)
    out, lse, routed = _routed_gpu(lay, q, t, idx, n_idx, lse0.cpu().double(), 0.65)
    lens = [n + t for n in lay.len0_host]
    c = oracle_cache(orc, lay, lens)
    _, _, er, margin = orc.sparse_routed(c, q, idx, n_idx, wl.n_recent, lse0.cpu().double(), 0.65)
    rg = routed.cpu().numpy()
    clear = np.abs(margin) > 1e-3
    assert (rg[clear] == er[clear]).all()
    frac = float(rg.mean())
    say(f"    groups routed: {int(rg.sum())} of {rg.size} ({100 * frac:.0f} %); "
        f"near-threshold: {int((~clear).sum())}")
    assert frac >= 0.5
    hm = torch.tensor(rg).repeat_interleave(wl.G, dim=1).to(torch.uint8)
    eo, el = orc.sparse(c, q, idx, n_idx, wl.n_recent, hm)
    assert_close_out(out.cpu().numpy(), eo, 1e-2)
    assert_close_rel(lse.cpu().numpy(), el, 1e-3, "lse")


@pytest.mark.parametrize("paged", [False, True])
def test_sparse_routed_edges(paged):
    """Lengths 0, 1 and 300: routing everything yields zeros (and no routing for the empty
    sequence); routing nothing is bit-identical to sfi_sparse_decode."""
    wl = synth.Workload("route_edges", 8300, 3, 16, 4, 128, "bf16", 300, 4, 32, 40, 2, sink=True,
                        paged=paged, block_size=16)
    lay = synth.make_layer(wl, 0, device=DEV, lens=[0, 1, 300])
    q = synth.make_query(wl, 0, 0, device=DEV, u=lay.u, n_for_sink=300)
    idx, n_idx = synth.synthetic_index_set(lay, "spans", seed=33)
    low = torch.full((wl.B, wl.Hq), -1e6, dtype=torch.float64)
    high = torch.full((wl.B, wl.Hq), 1e6, dtype=torch.float64)
    out, lse, routed = _routed_gpu(lay, q, 0, idx, n_idx, low, 0.65)
    assert routed.cpu().tolist() == [[0] * 4, [1] * 4, [1] * 4]
    assert (out == 0).all() and torch.isneginf(lse).all()
    out, lse, routed = _routed_gpu(lay, q, 0, idx, n_idx, high, 0.65)
    assert (routed == 0).all()
    ref_o, ref_l = gpu_sparse(lay, q, 0, idx.to(DEV), n_idx.to(DEV))
    assert torch.equal(out.nan_to_num(7.0), ref_o.nan_to_num(7.0))
    assert torch.equal(lse, ref_l)


def test_binding_rejects_misused_device_buffers():
    """The binding raises before the call for a wrong dtype or a strided view (cases chosen
    so that even an unchecked call would stay inside the tensors' storage)."""
    wl = W["gqa4_32k"].scaled(3000, B=1)
    lay = synth.make_layer(wl, 0, device=DEV)
    idx, n_idx = synth.synthetic_index_set(lay, "scattered", seed=23)
    idx, n_idx = idx.to(DEV), n_idx.to(DEV)
    lens = lay.len_at(1).to(DEV)
    desc = desc_for(lay, lens, lay.max_len_at(1))
    q = synth.make_query(wl, 0, 1, device=DEV)
    ws = B.workspace(desc, idx_stride=idx.shape[-1], n_recent=wl.n_recent, device=DEV)
    out64 = torch.zeros((wl.B, wl.Hq, wl.d), dtype=torch.float64, device=DEV)
    with pytest.raises(TypeError, match="out"):
        B.sfi_sparse_decode(desc, q, idx, idx.shape[-1], n_idx, wl.n_recent, None, out64, None, ws)
    wide = torch.zeros((wl.B, wl.Hkv, 2 * idx.shape[-1]), dtype=torch.int32, device=DEV)
    out = torch.zeros((wl.B, wl.Hq, wl.d), device=DEV)
    with pytest.raises(ValueError, match="contiguous"):
        B.sfi_sparse_decode(desc, q, wide[:, :, ::2], idx.shape[-1], n_idx, wl.n_recent, None,
                            out, None, ws)
    torch.cuda.synchronize()
    assert (out == 0).all(), "a rejected call must not have queued work"
