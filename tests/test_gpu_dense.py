"""Dense slow step on the GPU against the fp64 oracle (out, lse, fp32 logits)."""
import numpy as np
import pytest
import torch

from sparse_kv_attention_dense_amd import synth
from sparse_kv_attention_dense_amd import binding as B

from gpu_util import (DEV, assert_close_out, assert_close_rel, assert_logits, gpu_dense,
                      oracle_cache, say, tolerances, desc_for, workspace_for, round4)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
# Reduced contexts that keep each workload's structure, span several tiles and splits,
# and end in a ragged tail; the oracle finishes each in about a second.
SMALL = {
    "tiny_2k_f32": W["tiny_2k_f32"],
    "gqa4_32k": W["gqa4_32k"].scaled(5003),
    "sink_128k_b4": W["sink_128k_b4"].scaled(9001, B=2),
    "ragged_paged_b16": W["ragged_paged_b16"].scaled(6000, B=4, len_lo=2500),
    "gqa8_512k": W["gqa8_512k"].scaled(12007),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_dense_matches_oracle(orc, name):
    wl = SMALL[name]
    say(f"[dense] {wl.name} B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} d={wl.d} {wl.dtype} n0={wl.n0}")
    lay = synth.make_layer(wl, 0, device=DEV)
    q = synth.make_query(wl, 0, 0, device=DEV, u=lay.u)
    out, lse, logits, _ = gpu_dense(lay, q)
    eo, el, ez = orc.dense(oracle_cache(orc, lay, lay.len0_host), q)
    tol = tolerances(wl)
    assert_close_out(out.cpu().numpy(), eo, tol["out"])
    assert_close_rel(lse.cpu().numpy(), el, tol["rel"], "lse")
    assert_logits(logits, ez, lay.len0_host, tol["rel"])
    if wl.sink:
        p0 = np.exp(ez[:, :, 0] - el)
        say(f"    realised token-0 mass: mean {p0.mean():.3f}, range {p0.min():.3f}-{p0.max():.3f}")


@pytest.mark.parametrize("dtype,d,G", [("bf16", 64, 1), ("bf16", 128, 16), ("f32", 128, 2),
                                       ("bf16", 128, 3), ("bf16", 128, 5), ("bf16", 64, 7)])
def test_dense_head_shapes(orc, dtype, d, G):
    wl = synth.Workload(f"shape_{dtype}_{d}_{G}", 7100 + d + G, 2, 2 * G, 2, d, dtype, 1500,
                        4, 64, 128, 2)
    say(f"[dense] {wl.name}")
    lay = synth.make_layer(wl, 0, device=DEV, lens=[1500, 777])
    q = synth.make_query(wl, 0, 0, device=DEV)
    out, lse, logits, _ = gpu_dense(lay, q)
    eo, el, ez = orc.dense(oracle_cache(orc, lay, lay.len0_host), q)
    tol = tolerances(wl)
    assert_close_out(out.cpu().numpy(), eo, tol["out"])
    assert_close_rel(lse.cpu().numpy(), el, tol["rel"], "lse")
    assert_logits(logits, ez, lay.len0_host, tol["rel"])


@pytest.mark.parametrize("dtype,d,G,block", [("bf16", 128, 4, 1), ("bf16", 64, 8, 64),
                                             ("f32", 128, 2, 256), ("bf16", 128, 16, 1024)])
def test_dense_paged_page_sizes(orc, dtype, d, G, block):
    """Paged caches with pages of 1 to 1024 positions (block-table lookups per position, per
    page and spanning whole splits)."""
    wl = synth.Workload(f"dense_paged_{dtype}_{d}_{G}_{block}", 7200 + d + G + block, 2, 2 * G, 2,
                        d, dtype, 2600, 4, 64, 128, 2, paged=True, block_size=block)
    say(f"[dense] {wl.name}")
    lay = synth.make_layer(wl, 0, device=DEV, lens=[2600, 1333])
    q = synth.make_query(wl, 0, 0, device=DEV)
    out, lse, logits, _ = gpu_dense(lay, q)
    eo, el, ez = orc.dense(oracle_cache(orc, lay, lay.len0_host), q)
    tol = tolerances(wl)
    assert_close_out(out.cpu().numpy(), eo, tol["out"])
    assert_close_rel(lse.cpu().numpy(), el, tol["rel"], "lse")
    assert_logits(logits, ez, lay.len0_host, tol["rel"])


@pytest.mark.parametrize("case", range(10))
def test_dense_random_shapes(orc, case):
    """Seeded random dense steps against the oracle: batch 1-5 with lengths 0-20000 (a zero
    length on every third case with more than one sequence), 1-4 KV heads, groups of 1-16 query heads, d 64 or 128, bf16
    or fp32, a contiguous cache or pages of 1, 16 or 64 positions; out, lse and every logit
    below each length, and no logit written past it."""
    rng = np.random.default_rng(3000 + case)
    Bn = int(rng.integers(1, 6))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    block = int(rng.choice([0, 1, 16, 64]))
    lens = [int(x) for x in rng.integers(1, 20001, size=Bn)]
    if case % 3 == 0 and Bn > 1:                 # a whole batch of empty sequences has no
        lens[int(rng.integers(0, Bn))] = 0      # cache to point at (the ABI rejects that)
    wl = synth.Workload(f"dense_rand{case}", 9500 + case, Bn, Hkv * G, Hkv, d, dtype,
                        max(max(lens), 1), 4, 64, 128, 1, paged=block > 0,
                        block_size=max(block, 1))
    say(f"[dense random {case}] B={Bn} Hkv={Hkv} G={G} d={d} {dtype} block={block} lens={lens}")
    lay = synth.make_layer(wl, 0, device=DEV, lens=lens)
    q = synth.make_query(wl, 0, 0, device=DEV)
    out, lse, logits, _ = gpu_dense(lay, q)
    eo, el, ez = orc.dense(oracle_cache(orc, lay, lens), q)
    tol = tolerances(wl)
    assert_close_out(out.cpu().numpy(), eo, tol["out"])
    assert_close_rel(lse.cpu().numpy(), el, tol["rel"], "lse")
    assert_logits(logits, ez, lens, tol["rel"])
    lg = logits.cpu()
    for b, n in enumerate(lens):
        assert torch.isnan(lg[b, :, n:]).all(), "logits written past len"
        if n == 0:
            assert (out[b] == 0).all() and torch.isneginf(lse[b]).all()


def test_dense_loose_length_bound(orc):
    """max_len is only a host-side bound for the launch plan: a bound three times the longest
    sequence (as a captured step that must serve later, longer steps would declare) gives the
    same results against the oracle."""
    wl = synth.Workload("dense_loose_bound", 7350, 3, 16, 4, 128, "bf16", 6000, 4, 64, 128, 2)
    lay = synth.make_layer(wl, 0, device=DEV, lens=[6000, 2500, 777])
    q = synth.make_query(wl, 0, 0, device=DEV)
    lens = lay.len_at(0).to(DEV)
    stride = round4(3 * 6000)
    out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), device=DEV)
    lse = torch.full((wl.B, wl.Hq), float("nan"), device=DEV)
    logits = torch.full((wl.B, wl.Hq, stride), float("nan"), device=DEV)
    kbig = torch.zeros((wl.B, wl.Hkv, 3 * 6000, wl.d), dtype=lay.k.dtype, device=DEV)
    vbig = torch.zeros_like(kbig)
    kbig[:, :, :lay.k.shape[2]] = lay.k
    vbig[:, :, :lay.v.shape[2]] = lay.v
    desc = B.KVDesc(kbig, vbig, lens, 3 * 6000, wl.Hq)
    ws = B.workspace(desc, device=DEV)
    B.sfi_dense_decode(desc, q, out, lse, logits, stride, ws)
    torch.cuda.synchronize()
    eo, el, ez = orc.dense(oracle_cache(orc, lay, lay.len0_host), q)
    assert_close_out(out.cpu().numpy(), eo, 1e-2)
    assert_close_rel(lse.cpu().numpy(), el, 1e-3, "lse")
    assert_logits(logits, ez, lay.len0_host, 1e-3)


def test_dense_longest_single_unit_paged(orc):
    """One sequence, one KV head, 3M positions in 16-position pages: more positions than 1024
    splits of the default length cover, so the plan lengthens the splits (to 2944 positions)
    within the row table's capacity."""
    wl = synth.Workload("dense_3m_paged", 7500, 1, 2, 1, 64, "bf16", 3_000_000, 4, 64, 128, 1,
                        paged=True, block_size=16)
    say(f"[dense] {wl.name}")
    lay = synth.make_layer(wl, 0, device=DEV)
    q = synth.make_query(wl, 0, 0, device=DEV)
    out, lse, logits, _ = gpu_dense(lay, q)
    eo, el, ez = orc.dense(oracle_cache(orc, lay, lay.len0_host), q)
    assert_close_out(out.cpu().numpy(), eo, 1e-2)
    assert_close_rel(lse.cpu().numpy(), el, 1e-3, "lse")
    assert_logits(logits, ez, lay.len0_host, 1e-3)


def test_dense_edge_lengths(orc):
    """Lengths 0, 1, a tile minus one, a split plus one; logits past len stay untouched."""
    wl = synth.Workload("edges", 7300, 5, 8, 2, 128, "bf16", 4200, 4, 16, 32, 1)
    lens = [0, 1, 31, 129, 4200]
    lay = synth.make_layer(wl, 0, device=DEV, lens=lens)
    q = synth.make_query(wl, 0, 0, device=DEV)
    out, lse, logits, stride = gpu_dense(lay, q)
    eo, el, ez = orc.dense(oracle_cache(orc, lay, lens), q)
    assert (out[0] == 0).all() and torch.isneginf(lse[0]).all()
    assert_close_out(out.cpu().numpy(), eo, 1e-2)
    assert_close_rel(lse.cpu().numpy(), el, 1e-3, "lse")
    assert_logits(logits, ez, lens, 1e-3)
    lg = logits.cpu()
    for b, n in enumerate(lens):
        assert torch.isnan(lg[b, :, n:]).all(), "logits written past len"


def test_dense_without_logits_matches(orc):
    wl = SMALL["gqa4_32k"]
    lay = synth.make_layer(wl, 1, device=DEV)
    q = synth.make_query(wl, 1, 0, device=DEV)
    o1, l1, _, _ = gpu_dense(lay, q, logits=True)
    o2, l2, _, _ = gpu_dense(lay, q, logits=False)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_dense_deterministic():
    wl = SMALL["sink_128k_b4"]
    lay = synth.make_layer(wl, 2, device=DEV)
    q = synth.make_query(wl, 2, 0, device=DEV, u=lay.u)
    a = gpu_dense(lay, q)
    b = gpu_dense(lay, q)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x.nan_to_num(7.0), y.nan_to_num(7.0))


@pytest.mark.parametrize("name,samples", [("sink_128k_b4", [(0, 0), (3, 31), (1, 13)]),
                                          ("gqa8_512k", [(0, 0), (0, 63), (0, 22)]),
                                          ("ragged_paged_b16", [(0, 0), (7, 17), (15, 31)]),
                                          ("gqa4_32k", [(0, 5)])])
def test_dense_full_size_sampled(orc, name, samples):
    """Full-size workloads in the benchmark's launch configuration; the oracle recomputes
    sampled (batch, query head) rows one by one."""
    wl = W[name]
    say(f"[dense full] {wl.name} B={wl.B} n0={wl.n0}")
    lay = synth.make_layer(wl, 0, device=DEV)
    q = synth.make_query(wl, 0, 0, device=DEV, u=lay.u)
    out, lse, logits, _ = gpu_dense(lay, q)
    for b, i in samples:
        h = i // wl.G
        N = lay.len0_host[b]
        Kf, Vf = synth.logical_kv(lay, b, h, N)        # gathers through the block table when paged
        K1 = Kf.to(wl.torch_dtype)[None, None].contiguous()
        V1 = Vf.to(wl.torch_dtype)[None, None].contiguous()
        c = orc.Cache(K1, V1, torch.tensor([N], dtype=torch.int32), 1)
        eo, el, ez = orc.dense(c, q[b:b + 1, i:i + 1].contiguous())
        say(f"  sample b={b} i={i}")
        assert_close_out(out[b, i].cpu().numpy()[None, None], eo, 1e-2)
        assert_close_rel(lse[b, i:i + 1].cpu().numpy()[None], el, 1e-3, "lse")
        assert_logits(logits[b:b + 1, i:i + 1], ez, [N], 1e-3)
    del lay, out, logits
    torch.cuda.empty_cache()
