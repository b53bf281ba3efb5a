"""Pins for the fp64 CPU oracle, checked against things other than the oracle itself.

* dense attention against torch's scaled_dot_product_attention in float64 (a library
  routine) and closed forms (one token, identical keys, zero query, zero-norm sink,
  weights summing to one, permutation invariance, exact integer logits, a hand-derived
  golden case);
* the selector against planted rankings known by construction, the identity when the
  budget covers J, a library sort when the group has one head, brute-force rank
  counting with ties, and a hand-derived case for the per-head normalisation over J;
* the sparse step against the library attention with a boolean mask, the dense result
  when the set is everything, and the zero surrogate;
* the Reorg and the two-segment step: segment rows against the cache rows read by tensor
  indexing, exact agreement with the gather step on the same index set, snapshot semantics
  against the library attention on the original rows;
* the sink-bypass mask against a library sort;
* the full Selector (prior, fusion, Soft-NMS, cross-head exclusivity: readings of lost
  equations): its reduction to the plain Selector, the fusion against a numerical minimum of
  its defining objective, scale invariance and monotonicity of the key-norm factor, the
  position factor's closed form, Soft-NMS against a library maximum filter, exclusivity under
  a permutation of the heads, and two hand-derived golden cases.
No test here needs a GPU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from sparse_kv_attention_dense_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _cache(orc, K, V, lens, Hq, **kw):
    return orc.Cache(K, V, torch.tensor(lens, dtype=torch.int32), Hq, **kw)


def _sdpa_ref(q, Kl, Vl, mask=None):
    """Library attention (float64) for one sequence: q [Hq][d], K/V [Hkv][n][d]."""
    Hq, Hkv = q.shape[0], Kl.shape[0]
    G = Hq // Hkv
    k = Kl.double().repeat_interleave(G, dim=0)
    v = Vl.double().repeat_interleave(G, dim=0)
    qq = q.double()[:, None, :]
    am = None if mask is None else mask.repeat_interleave(G, dim=0)[:, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qq, k, v, attn_mask=am)[:, 0]
    z = (qq @ k.transpose(1, 2))[:, 0] / math.sqrt(q.shape[-1])
    if mask is not None:
        z = z.masked_fill(~mask.repeat_interleave(G, dim=0), -math.inf)
    return out, torch.logsumexp(z, dim=-1), (qq @ k.transpose(1, 2))[:, 0] / math.sqrt(q.shape[-1])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("Hq,Hkv,d", [(4, 1, 16), (4, 2, 8), (8, 4, 32), (6, 3, 64)])
def test_dense_matches_library_attention(orc, dtype, Hq, Hkv, d):
    g = torch.Generator().manual_seed(Hq * 100 + d)
    B, cap = 3, 70
    lens = [1, 37, 70]
    K = torch.randn((B, Hkv, cap, d), generator=g).to(dtype)
    V = torch.randn((B, Hkv, cap, d), generator=g).to(dtype)
    q = torch.randn((B, Hq, d), generator=g).to(dtype)
    out, lse, logits = orc.dense(_cache(orc, K, V, lens, Hq), q, logit_stride=cap)
    for b in range(B):
        n = lens[b]
        ro, rl, rz = _sdpa_ref(q[b], K[b, :, :n], V[b, :, :n])
        np.testing.assert_allclose(out[b], ro.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], rl.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(logits[b, :, :n], rz.numpy(), rtol=0, atol=1e-12)


def test_dense_paged_matches_contiguous_library(orc):
    """Paged cache read through a shuffled block table equals the logical sequence."""
    wl = synth.Workload("paged_tiny", 77, 3, 8, 2, 32, "bf16", 90, 4, 8, 16, 3, paged=True,
                        block_size=16, len_lo=20)
    lay = synth.make_layer(wl, 0)
    q = synth.make_query(wl, 0, 0)
    c = orc.Cache(lay.k, lay.v, lay.len0, wl.Hq, block_table=lay.block_table,
                  block_size=wl.block_size, max_blocks=lay.max_blocks)
    out, lse, logits = orc.dense(c, q, logit_stride=lay.cap)
    for b in range(wl.B):
        n = lay.len0_host[b]
        Ks, Vs = zip(*[synth.logical_kv(lay, b, h, n) for h in range(wl.Hkv)])
        ro, rl, rz = _sdpa_ref(q[b].float(), torch.stack(Ks), torch.stack(Vs))
        np.testing.assert_allclose(out[b], ro.numpy(), atol=1e-12)
        np.testing.assert_allclose(lse[b], rl.numpy(), atol=1e-12)
        np.testing.assert_allclose(logits[b, :, :n], rz.numpy(), atol=1e-12)


def test_dense_golden_two_token(orc):
    gd = json.load(open(os.path.join(HERE, "golden", "dense_two_token.json")))
    K = torch.tensor(gd["k"], dtype=torch.float32)[None, None]
    V = torch.tensor(gd["v"], dtype=torch.float32)[None, None]
    q = torch.tensor(gd["q"], dtype=torch.float32)[None, None]
    out, lse, logits = orc.dense(_cache(orc, K, V, [2], 1), q)
    tol = gd["tolerance"]
    np.testing.assert_allclose(logits[0, 0, :2], gd["expected_logits"], atol=tol)
    assert abs(lse[0, 0] - gd["expected_lse"]) < tol
    np.testing.assert_allclose(out[0, 0], gd["expected_out"], atol=tol)


def test_dense_closed_forms(orc):
    g = torch.Generator().manual_seed(5)
    d, n = 16, 50
    K = torch.randn((1, 1, n, d), generator=g)
    V = torch.randn((1, 1, n, d), generator=g)
    q = torch.randn((1, 2, d), generator=g)
    # one token: out = v0, lse = z0
    out, lse, z = orc.dense(_cache(orc, K, V, [1], 2), q)
    np.testing.assert_allclose(out[0, 0], V[0, 0, 0].double().numpy(), atol=1e-14)
    assert abs(lse[0, 1] - z[0, 1, 0]) < 1e-14
    # identical keys: uniform weights -> mean of V, lse = z + ln n
    Ks = K[:, :, :1].expand(1, 1, n, d).contiguous()
    out, lse, z = orc.dense(_cache(orc, Ks, V, [n], 2), q)
    np.testing.assert_allclose(out[0, 0], V[0, 0].double().mean(0).numpy(), atol=1e-12)
    assert abs(lse[0, 0] - (z[0, 0, 0] + math.log(n))) < 1e-12
    # zero query: lse = ln n, out = mean of V
    out, lse, _ = orc.dense(_cache(orc, K, V, [n], 2), torch.zeros((1, 2, d)))
    assert abs(lse[0, 0] - math.log(n)) < 1e-13
    np.testing.assert_allclose(out[0, 1], V[0, 0].double().mean(0).numpy(), atol=1e-12)
    # weights sum to one: sum_j exp(z_j - lse) = 1
    out, lse, z = orc.dense(_cache(orc, K, V, [n], 2), q)
    assert abs(np.exp(z[0, 0, :n] - lse[0, 0]).sum() - 1.0) < 1e-12


def test_dense_zero_norm_sink(orc):
    """v0 = 0: out = (1 - p0) * (attention over positions >= 1)."""
    g = torch.Generator().manual_seed(6)
    d, n = 32, 40
    K = torch.randn((1, 1, n, d), generator=g)
    V = torch.randn((1, 1, n, d), generator=g)
    V[0, 0, 0] = 0
    q = torch.randn((1, 1, d), generator=g)
    out, lse, z = orc.dense(_cache(orc, K, V, [n], 1), q)
    p0 = math.exp(z[0, 0, 0] - lse[0, 0])
    out_rest, _, _ = orc.dense(_cache(orc, K[:, :, 1:].contiguous(), V[:, :, 1:].contiguous(),
                                      [n - 1], 1), q)
    np.testing.assert_allclose(out[0, 0], (1 - p0) * out_rest[0, 0], atol=1e-13)


def test_dense_permutation_invariance(orc):
    g = torch.Generator().manual_seed(7)
    d, n = 16, 33
    K = torch.randn((1, 2, n, d), generator=g)
    V = torch.randn((1, 2, n, d), generator=g)
    q = torch.randn((1, 4, d), generator=g)
    perm = torch.randperm(n, generator=g)
    o1, l1, z1 = orc.dense(_cache(orc, K, V, [n], 4), q)
    o2, l2, z2 = orc.dense(_cache(orc, K[:, :, perm].contiguous(), V[:, :, perm].contiguous(),
                                  [n], 4), q)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    np.testing.assert_allclose(z1[:, :, perm.numpy()], z2, atol=0)


def test_dense_exact_integer_logits_and_group_map(orc):
    """Small-integer q and k make every logit exact: z = (q.k)/8 at d = 64.  Query head i
    must read KV head i // G (here G = 2, KV heads 0..2 hold different keys)."""
    g = torch.Generator().manual_seed(8)
    d, n, Hkv, G = 64, 9, 3, 2
    K = torch.randint(-3, 4, (1, Hkv, n, d), generator=g).float()
    V = torch.randn((1, Hkv, n, d), generator=g)
    q = torch.randint(-3, 4, (1, Hkv * G, d), generator=g).float()
    _, _, z = orc.dense(_cache(orc, K, V, [n], Hkv * G), q)
    for i in range(Hkv * G):
        for j in range(n):
            exact = sum(int(a) * int(b) for a, b in zip(q[0, i], K[0, i // G, j])) / 8.0
            assert z[0, i, j] == exact


# ---------------------------------------------------------------------------- selector

def _expected_from_ranks(ranks, lens, n_sink, n_recent, k_sel, Hkv):
    exp = []
    for b, rb in enumerate(ranks):
        N = int(lens[b])
        ns = min(n_sink, N)
        row = []
        for h in range(Hkv):
            pi = rb[h]
            J_lo = n_sink
            keep = sorted((torch.nonzero(pi < k_sel).flatten() + J_lo).tolist())
            row.append(list(range(ns)) + keep)
        exp.append(row)
    return exp


@pytest.mark.parametrize("G,lens,k_sel", [(4, [300, 257, 1000], 64), (1, [500], 37),
                                          (8, [2000, 2000], 511)])
def test_select_planted_ranks(orc, G, lens, k_sel):
    Hkv, n_sink, n_recent = 2, 4, 16
    Hq = Hkv * G
    stride = max(lens)
    z, ranks = synth.planted_logits(len(lens), Hq, Hkv, lens, n_sink, n_recent, stride,
                                    seed=11 + G, noise_sink=40.0)
    idx, n_idx, f = orc.select(lens, Hq, Hkv, z, n_sink, n_recent, k_sel, want_f=True)
    exp = _expected_from_ranks(ranks, lens, n_sink, n_recent, k_sel, Hkv)
    for b in range(len(lens)):
        for h in range(Hkv):
            got = idx[b, h, :n_idx[b, h]].tolist()
            assert got == exp[b][h]
            N = lens[b]
            assert abs(f[b, h, n_sink:N - n_recent].sum() - 1.0) < 1e-12
            assert (f[b, h, :n_sink] == 0).all() and (f[b, h, N - n_recent:] == 0).all()


def test_select_budget_covers_J_is_identity(orc):
    lens = [100, 40, 3]
    Hq, Hkv, n_sink, n_recent = 4, 2, 4, 16
    z = torch.randn((3, Hq, 100), generator=torch.Generator().manual_seed(3))
    idx, n_idx, _ = orc.select(lens, Hq, Hkv, z, n_sink, n_recent, k_sel=200,
                               idx_stride=300)
    for b, N in enumerate(lens):
        J = list(range(n_sink, max(n_sink, N - n_recent)))
        for h in range(Hkv):
            assert idx[b, h, :n_idx[b, h]].tolist() == list(range(min(n_sink, N))) + J


def test_select_single_head_is_library_topk(orc):
    """G = 1: f is the softmax over J, monotone in z, so the choice is a plain sort of z
    (numpy lexsort: z descending, position ascending)."""
    g = torch.Generator().manual_seed(4)
    N, n_sink, n_recent, k_sel = 700, 4, 32, 50
    z = torch.randint(-20, 20, (1, 3, N), generator=g).float() / 4   # many exact ties
    idx, n_idx, _ = orc.select([N], 3, 3, z, n_sink, n_recent, k_sel)
    for h in range(3):
        zJ = z[0, h, n_sink:N - n_recent].double().numpy()
        pos = np.arange(n_sink, N - n_recent)
        order = np.lexsort((pos, -zJ))[:k_sel]
        exp = list(range(n_sink)) + sorted(pos[order].tolist())
        assert idx[0, h, :n_idx[0, h]].tolist() == exp


def test_select_observation_window_is_the_mean_over_queries(orc):
    """Evidence over a window of W queries per head (rows i*W + w of the logits, so KV head h
    owns G*W rows) is the mean of the W single-query evidences, each over its G rows; a window
    of W copies of one query gives that query's evidence and selection."""
    g = torch.Generator().manual_seed(12)
    B, Hq, Hkv, Wn, N = 2, 8, 2, 4, 600
    n_sink, n_recent, k_sel = 4, 40, 90
    lens = [N, 437]
    z = torch.randn((B, Hq * Wn, N), generator=g) * 2.0
    _, _, fw = orc.select(lens, Hq * Wn, Hkv, z, n_sink, n_recent, k_sel, want_f=True)
    f_each = []
    for w in range(Wn):
        _, _, f = orc.select(lens, Hq, Hkv, z[:, w::Wn], n_sink, n_recent, k_sel, want_f=True)
        f_each.append(f)
    for b, n in enumerate(lens):
        J = slice(n_sink, n - n_recent)
        mean = sum(f[b][:, J] for f in f_each) / Wn
        assert np.allclose(fw[b][:, J], mean, rtol=1e-12, atol=0.0)
    z1 = torch.randn((B, Hq, N), generator=g)
    i1, n1, _ = orc.select(lens, Hq, Hkv, z1, n_sink, n_recent, k_sel)
    iw, nw, _ = orc.select(lens, Hq * Wn, Hkv, z1.repeat_interleave(Wn, dim=1), n_sink, n_recent,
                           k_sel)
    assert (n1 == nw).all() and (i1 == iw).all()


def test_select_brute_force_rank_counting(orc):
    """O(n^2) rank counting on tiny inputs with ties: j is kept iff fewer than k_sel
    positions beat it ((f larger) or (f equal and position lower))."""
    g = torch.Generator().manual_seed(9)
    N, n_sink, n_recent, k_sel, Hq, Hkv = 60, 3, 5, 17, 4, 2
    z = torch.randint(-3, 3, (2, Hq, N), generator=g).double()
    idx, n_idx, f = orc.select([N, N - 7], Hq, Hkv, z, n_sink, n_recent, k_sel, want_f=True)
    for b, Nb in enumerate([N, N - 7]):
        for h in range(Hkv):
            J = range(n_sink, Nb - n_recent)
            fb = f[b, h]
            keep = [j for j in J
                    if sum(1 for j2 in J if fb[j2] > fb[j] or (fb[j2] == fb[j] and j2 < j))
                    < k_sel]
            assert idx[b, h, :n_idx[b, h]].tolist() == list(range(n_sink)) + keep


def test_select_ignores_sink_and_recent_logits(orc):
    lens = [400]
    Hq, Hkv, n_sink, n_recent, k_sel = 4, 1, 4, 64, 30
    z = torch.randn((1, Hq, 400), generator=torch.Generator().manual_seed(12))
    a, _, _ = orc.select(lens, Hq, Hkv, z, n_sink, n_recent, k_sel)
    z2 = z.clone()
    z2[:, :, :n_sink] = 1e4
    z2[:, :, 400 - n_recent:] = -1e4
    z2[:, 1, 400 - n_recent:] = 1e4
    b, _, _ = orc.select(lens, Hq, Hkv, z2, n_sink, n_recent, k_sel)
    assert (a == b).all()


def test_select_golden_normalisation_over_J(orc):
    gd = json.load(open(os.path.join(HERE, "golden", "select_lse_j.json")))
    N = gd["N"]
    z = torch.tensor([[gd["z_head0"], gd["z_head1"]]], dtype=torch.float64)
    idx, n_idx, f = orc.select([N], 2, 1, z, gd["n_sink"], gd["n_recent"], gd["k_sel"],
                               want_f=True)
    assert idx[0, 0, :n_idx[0, 0]].tolist() == gd["expected_idx"]
    for j, v in gd["expected_f_at"].items():
        assert abs(f[0, 0, int(j)] - v) < gd["tolerance"]


def test_select_short_contexts(orc):
    """N - n_recent <= n_sink: J is empty and only the sinks come back; N < n_sink: [0, N)."""
    z = torch.randn((3, 2, 30), generator=torch.Generator().manual_seed(2))
    idx, n_idx, _ = orc.select([30, 12, 2], 2, 1, z, n_sink=4, n_recent=26, k_sel=8)
    assert idx[0, 0, :n_idx[0, 0]].tolist() == [0, 1, 2, 3]
    assert idx[1, 0, :n_idx[1, 0]].tolist() == [0, 1, 2, 3]
    assert idx[2, 0, :n_idx[2, 0]].tolist() == [0, 1]


# ------------------------------------------------------------------------------ sparse

@pytest.mark.parametrize("paged", [False, True])
def test_sparse_matches_library_masked_attention(orc, paged):
    wl = synth.Workload("sp_tiny", 91, 2, 8, 2, 32, "bf16", 300, 4, 20, 40, 3, paged=paged,
                        block_size=16, len_lo=150 if paged else 0)
    lay = synth.make_layer(wl, 0)
    q = synth.make_query(wl, 0, 1)
    lens = [n + 1 for n in lay.len0_host]          # one fast step after the slow step
    idx, n_idx = synth.synthetic_index_set(lay, "spans", seed=5)
    kw = dict(block_table=lay.block_table, block_size=wl.block_size,
              max_blocks=lay.max_blocks) if paged else {}
    c = orc.Cache(lay.k, lay.v, torch.tensor(lens, dtype=torch.int32), wl.Hq, **kw)
    out, lse = orc.sparse(c, q, idx, n_idx, wl.n_recent)
    for b in range(wl.B):
        N = lens[b]
        Ks, Vs = zip(*[synth.logical_kv(lay, b, h, N) for h in range(wl.Hkv)])
        mask = torch.zeros((wl.Hkv, N), dtype=torch.bool)
        for h in range(wl.Hkv):
            sel = idx[b, h, :n_idx[b, h]].long()
            mask[h, sel[sel < N - wl.n_recent]] = True
            mask[h, max(0, N - wl.n_recent):] = True
        ro, rl, _ = _sdpa_ref(q[b].float(), torch.stack(Ks), torch.stack(Vs), mask)
        np.testing.assert_allclose(out[b], ro.numpy(), atol=1e-12)
        np.testing.assert_allclose(lse[b], rl.numpy(), atol=1e-12)


def test_sparse_full_set_equals_dense_and_mask_zero(orc):
    g = torch.Generator().manual_seed(13)
    d, n, Hq, Hkv, n_recent = 16, 80, 4, 2, 10
    K = torch.randn((1, Hkv, n, d), generator=g)
    V = torch.randn((1, Hkv, n, d), generator=g)
    q = torch.randn((1, Hq, d), generator=g)
    c = _cache(orc, K, V, [n], Hq)
    od, ld, _ = orc.dense(c, q)
    full = torch.arange(n - n_recent, dtype=torch.int32).repeat(1, Hkv, 1)
    os_, ls, = orc.sparse(c, q, full, torch.full((1, Hkv), n - n_recent, dtype=torch.int32),
                          n_recent)
    np.testing.assert_allclose(os_, od, atol=1e-13)
    np.testing.assert_allclose(ls, ld, atol=1e-13)
    # entries in the recent window or beyond the length are ignored; repeats count once
    noisy = torch.cat([full, full[:, :, :5], torch.full((1, Hkv, 4), n + 3, dtype=torch.int32)],
                      dim=2)
    on, _ = orc.sparse(c, q, noisy, torch.full((1, Hkv), noisy.shape[-1], dtype=torch.int32),
                       n_recent)
    np.testing.assert_allclose(on, od, atol=1e-13)
    # empty selection: window attention over the last n_recent positions
    ow, lw = orc.sparse(c, q, full, torch.zeros((1, Hkv), dtype=torch.int32), n_recent)
    cw = _cache(orc, K[:, :, n - n_recent:].contiguous(), V[:, :, n - n_recent:].contiguous(),
                [n_recent], Hq)
    ow2, lw2, _ = orc.dense(cw, q)
    np.testing.assert_allclose(ow, ow2, atol=1e-13)
    # a masked head outputs exact zeros
    hm = torch.tensor([[0, 1, 0, 1]], dtype=torch.uint8)
    om, lm = orc.sparse(c, q, full, torch.full((1, Hkv), n - n_recent, dtype=torch.int32),
                        n_recent, head_mask=hm)
    assert (om[0, 1] == 0).all() and (om[0, 3] == 0).all() and np.isneginf(lm[0, 1])
    np.testing.assert_allclose(om[0, 0], od[0, 0], atol=1e-13)


# ------------------------------------------------------- reorg and the two-segment step

def _as_f32(rows):
    """Segment rows (bf16 bits as uint16, or float32) as float32 values."""
    if rows.dtype == np.uint16:
        return (rows.astype(np.uint32) << 16).view(np.float32)
    return rows


def _two_segment_case(paged, seed=21):
    wl = synth.Workload("ts_tiny", 95, 2, 8, 2, 32, "bf16", 300, 4, 20, 40, 6, paged=paged,
                        block_size=16, len_lo=150 if paged else 0)
    lay = synth.make_layer(wl, 0)
    idx, n_idx = synth.synthetic_index_set(lay, "scattered", seed=seed)
    return wl, lay, idx, n_idx


def _orc_cache(orc, wl, lay, lens):
    kw = dict(block_table=lay.block_table, block_size=wl.block_size,
              max_blocks=lay.max_blocks) if wl.paged else {}
    return orc.Cache(lay.k, lay.v, torch.tensor(lens, dtype=torch.int32), wl.Hq, **kw)


@pytest.mark.parametrize("paged", [False, True])
def test_reorg_rows_are_the_cache_rows(orc, paged):
    wl, lay, idx, n_idx = _two_segment_case(paged)
    lens = lay.len0_host
    idx = idx.clone()
    idx[0, 0, 3] = -3                               # outside the sequence: zero rows, cpos -1
    idx[1, 1, 5] = lens[1] + 2
    n_idx = n_idx.clone()
    n_idx[0, 1] -= 7                                # slots past the count: zero rows, cpos -1
    ck, cv, cpos = orc.reorg(_orc_cache(orc, wl, lay, lens), idx, n_idx)
    for b in range(wl.B):
        for h in range(wl.Hkv):
            Kl, Vl = synth.logical_kv(lay, b, h, lens[b])
            for s in range(idx.shape[-1]):
                p = int(idx[b, h, s])
                if s < int(n_idx[b, h]) and 0 <= p < lens[b]:
                    assert cpos[b, h, s] == p
                    np.testing.assert_array_equal(_as_f32(ck[b, h, s]), Kl[p].numpy())
                    np.testing.assert_array_equal(_as_f32(cv[b, h, s]), Vl[p].numpy())
                else:
                    assert cpos[b, h, s] == -1
                    assert not ck[b, h, s].any() and not cv[b, h, s].any()


@pytest.mark.parametrize("paged", [False, True])
def test_two_segment_step_equals_gather_step(orc, paged):
    wl, lay, idx, n_idx = _two_segment_case(paged)
    ck, cv, cpos = orc.reorg(_orc_cache(orc, wl, lay, lay.len0_host), idx, n_idx)
    hm = torch.zeros((wl.B, wl.Hq), dtype=torch.uint8)
    hm[1, 2] = 1
    for t in (1, 3, 5):                             # the recent window moves; the segment stays
        lens = [n + t for n in lay.len0_host]
        c = _orc_cache(orc, wl, lay, lens)
        q = synth.make_query(wl, 0, t)
        og, lg = orc.sparse(c, q, idx, n_idx, wl.n_recent, head_mask=hm)
        oc, lc = orc.sparse_compact(c, q, ck, cv, cpos, n_idx, wl.n_recent, head_mask=hm)
        np.testing.assert_array_equal(oc, og)
        np.testing.assert_array_equal(lc, lg)
        assert (oc[1, 2] == 0).all() and np.isneginf(lc[1, 2])


def test_two_segment_step_reads_the_snapshot(orc):
    wl, lay, idx, n_idx = _two_segment_case(False)
    lens0 = lay.len0_host
    ck, cv, cpos = orc.reorg(_orc_cache(orc, wl, lay, lens0), idx, n_idx)
    K0, V0 = lay.k.clone(), lay.v.clone()
    # overwrite the cache rows of some selected positions after the Reorg
    g = torch.Generator().manual_seed(3)
    for b in range(wl.B):
        for h in range(wl.Hkv):
            for p in idx[b, h, wl.n_sink:wl.n_sink + 6].tolist():
                lay.k[b, h, p] = torch.randn(wl.d, generator=g).to(lay.k.dtype)
                lay.v[b, h, p] = torch.randn(wl.d, generator=g).to(lay.v.dtype)
    t = 2
    lens = [n + t for n in lens0]
    q = synth.make_query(wl, 0, t)
    oc, lc = orc.sparse_compact(_orc_cache(orc, wl, lay, lens), q, ck, cv, cpos, n_idx,
                                wl.n_recent)
    og, _ = orc.sparse(_orc_cache(orc, wl, lay, lens), q, idx, n_idx, wl.n_recent)
    assert np.abs(oc - og).max() > 1e-3            # the gather step sees the new rows
    for b in range(wl.B):                           # the segment holds the rows of the Reorg
        N = lens[b]
        mask = torch.zeros((wl.Hkv, N), dtype=torch.bool)
        for h in range(wl.Hkv):
            sel = idx[b, h, :n_idx[b, h]].long()
            mask[h, sel[sel < N - wl.n_recent]] = True
            mask[h, N - wl.n_recent:] = True
        ro, rl, _ = _sdpa_ref(q[b].float(), K0[b, :, :N].float(), V0[b, :, :N].float(), mask)
        np.testing.assert_allclose(oc[b], ro.numpy(), atol=1e-12)
        np.testing.assert_allclose(lc[b], rl.numpy(), atol=1e-12)


def test_two_segment_drops_entries_past_the_reorg_length(orc):
    wl, lay, idx, n_idx = _two_segment_case(False)
    lens0 = lay.len0_host
    # the Reorg sees shorter sequences: entries at or past its length are dropped, although
    # the fast step's cache holds those positions below its recent window
    short = [n - 100 for n in lens0]
    dropped = sum(int(((idx[b, :, :] >= short[b]) & (idx[b] < lens0[b] - wl.n_recent)).sum())
                  for b in range(wl.B))
    assert dropped > 0
    ck, cv, cpos = orc.reorg(_orc_cache(orc, wl, lay, short), idx, n_idx)
    lens = [n + 1 for n in lens0]
    q = synth.make_query(wl, 0, 1)
    c = _orc_cache(orc, wl, lay, lens)
    oc, lc = orc.sparse_compact(c, q, ck, cv, cpos, n_idx, wl.n_recent)
    kept = idx.clone()
    for b in range(wl.B):
        kept[b][kept[b] >= short[b]] = -1           # the gather step skips negative entries
    og, lg = orc.sparse(c, q, kept, n_idx, wl.n_recent)
    np.testing.assert_array_equal(oc, og)
    np.testing.assert_array_equal(lc, lg)


# ----------------------------------------------------------------- the full Selector

NOREF = dict(lambda_=0.0, alpha_soft=0.0, alpha_cross=0.0)


@pytest.mark.parametrize("B,Hq,Hkv,lens,k_sel", [(2, 8, 2, [700, 333], 50), (1, 4, 4, [260], 7),
                                                 (3, 6, 3, [40, 1, 500], 30)])
def test_refined_reduces_to_selector(orc, B, Hq, Hkv, lens, k_sel):
    g = np.random.default_rng(5)
    z = g.normal(size=(B, Hq, max(lens))) * 2.0
    kn = g.uniform(0.5, 2.0, size=(B, Hkv, max(lens)))
    a, na, _ = orc.select(lens, Hq, Hkv, z, 4, 16, k_sel)
    b, nb, _, _ = orc.select_refined(lens, Hq, Hkv, z, 4, 16, k_sel, key_norm=kn, params=NOREF)
    assert (a == b).all() and (na == nb).all()
    # a uniform prior with lambda > 0 keeps the order of the evidence (s ~ f^(1-lambda))
    flat = dict(lambda_=0.02, alpha_soft=0.0, alpha_cross=0.0, prior_decay=0.0, tail_brake=0.0)
    c, nc, _, _ = orc.select_refined(lens, Hq, Hkv, z, 4, 16, k_sel, params=flat)
    assert (a == c).all() and (na == nc).all()


def test_fusion_minimises_the_kl_objective(orc):
    from scipy.optimize import minimize
    g = np.random.default_rng(6)
    N, n_sink, n_recent, Hq = 14, 2, 2, 2                     # J = [2, 12), G = 2
    z = g.normal(size=(1, Hq, N)) * 1.5
    kn = g.uniform(0.5, 2.0, size=(1, 1, N))
    base = dict(alpha_soft=0.0, alpha_cross=0.0, prior_decay=1.3, tail_frac=0.25, tail_brake=2.0)
    _, _, f = orc.select([N], Hq, 1, z, n_sink, n_recent, 3, want_f=True)
    fJ = f[0, 0, n_sink:N - n_recent]
    # lambda = 1: the fused distribution is the prior itself
    _, _, fr, _ = orc.select_refined([N], Hq, 1, z, n_sink, n_recent, 3, key_norm=kn,
                                     params=dict(base, lambda_=1.0), want_scores=True)
    r = np.exp(fr[0, 0, n_sink:N - n_recent])
    assert abs(r.sum() - 1.0) < 1e-12
    lam = 0.3
    _, _, fs, _ = orc.select_refined([N], Hq, 1, z, n_sink, n_recent, 3, key_norm=kn,
                                     params=dict(base, lambda_=lam), want_scores=True)
    s = np.exp(fs[0, 0, n_sink:N - n_recent])

    def objective(x):
        q = np.exp(x - x.max())
        q /= q.sum()
        return (1 - lam) * np.sum(q * np.log(q / fJ)) + lam * np.sum(q * np.log(q / r))

    res = minimize(objective, np.log(fJ), method="BFGS", options=dict(gtol=1e-12))
    q = np.exp(res.x - res.x.max())
    q /= q.sum()
    np.testing.assert_allclose(s, q, atol=1e-6)
    assert objective(np.log(s)) <= res.fun + 1e-12


def test_prior_key_norm_and_position_factors(orc):
    g = np.random.default_rng(7)
    N, n_sink, n_recent, Hq, Hkv = 200, 4, 20, 4, 2
    z = g.normal(size=(1, Hq, N))
    kn = g.uniform(0.5, 2.0, size=(1, Hkv, N))
    prm = dict(lambda_=0.02, alpha_soft=0.0, alpha_cross=0.0)
    _, _, f1, _ = orc.select_refined([N], Hq, Hkv, z, n_sink, n_recent, 5, key_norm=kn,
                                     params=prm, want_scores=True)
    _, _, f3, _ = orc.select_refined([N], Hq, Hkv, z, n_sink, n_recent, 5, key_norm=3 * kn,
                                     params=prm, want_scores=True)
    J = slice(n_sink, N - n_recent)
    np.testing.assert_allclose(f1[:, :, J], f3[:, :, J], atol=1e-12)     # only ratios matter
    kn2 = kn.copy()
    kn2[0, 0, 50] *= 4.0                                                  # a longer key
    _, _, f4, _ = orc.select_refined([N], Hq, Hkv, z, n_sink, n_recent, 5, key_norm=kn2,
                                     params=prm, want_scores=True)
    assert f4[0, 0, 50] < f1[0, 0, 50]
    others = np.delete(np.arange(n_sink, N - n_recent), 50 - n_sink)
    assert (f4[0, 0, others] > f1[0, 0, others]).all()
    np.testing.assert_allclose(f4[0, 1, J], f1[0, 1, J], atol=1e-12)     # the other head
    # position factor on uniform evidence with lambda = 1 (s is the prior): consecutive
    # log-ratios are -decay/|J| before the tail and -(decay + brake/tail_frac)/|J| inside it
    nJ = N - n_recent - n_sink
    pos = dict(lambda_=1.0, alpha_soft=0.0, alpha_cross=0.0, prior_decay=0.7, tail_frac=0.25,
               tail_brake=1.5)
    _, _, fu, _ = orc.select_refined([N], Hq, Hkv, np.zeros((1, Hq, N)), n_sink, n_recent, 5,
                                     params=pos, want_scores=True)
    d = np.diff(fu[0, 0, J])
    u = (np.arange(nJ) + 0.5) / nJ
    body = (u[1:] <= 0.75)
    tail = (u[:-1] >= 0.75)
    np.testing.assert_allclose(d[body], -0.7 / nJ, atol=1e-12)
    np.testing.assert_allclose(d[tail], -(0.7 + 1.5 / 0.25) / nJ, atol=1e-12)


def test_soft_nms_golden(orc):
    gd = json.load(open(os.path.join(HERE, "golden", "select_soft_nms.json")))
    z = np.array([[gd["z"]]])
    plain, _, _ = orc.select([gd["N"]], 1, 1, z, gd["n_sink"], gd["n_recent"], gd["k_sel"])
    assert plain[0, 0].tolist() == gd["expected_idx_plain"]
    prm = dict(lambda_=0.0, alpha_soft=gd["alpha_soft"], alpha_cross=0.0)
    idx, n_idx, _, ref = orc.select_refined([gd["N"]], 1, 1, z, gd["n_sink"], gd["n_recent"],
                                            gd["k_sel"], params=prm, want_scores=True)
    assert idx[0, 0, :n_idx[0, 0]].tolist() == gd["expected_idx"]
    np.testing.assert_allclose(ref[0, 0], gd["expected_refined"], atol=gd["tolerance"])


def test_cross_head_golden(orc):
    gd = json.load(open(os.path.join(HERE, "golden", "select_cross_head.json")))
    z = np.array([[gd["z_head0"], gd["z_head1"]]])
    plain, _, _ = orc.select([gd["N"]], 2, 2, z, gd["n_sink"], gd["n_recent"], gd["k_sel"])
    assert plain[0].tolist() == gd["expected_idx_plain"]
    prm = dict(lambda_=0.0, alpha_soft=0.0, alpha_cross=gd["alpha_cross"])
    idx, _, _, ref = orc.select_refined([gd["N"]], 2, 2, z, gd["n_sink"], gd["n_recent"],
                                        gd["k_sel"], params=prm, want_scores=True)
    assert idx[0].tolist() == gd["expected_idx"]
    np.testing.assert_allclose(ref[0], gd["expected_refined"], atol=gd["tolerance"])


def test_soft_nms_matches_a_library_maximum_filter(orc):
    from scipy.ndimage import maximum_filter1d
    g = np.random.default_rng(8)
    N, n_sink, n_recent = 300, 4, 30
    z = np.round(g.normal(size=(1, 2, N)) * 4) / 4            # exact ties between neighbours
    prm = dict(lambda_=0.02, alpha_soft=0.5, alpha_cross=0.0)
    _, _, fused, ref = orc.select_refined([N], 2, 1, z, n_sink, n_recent, 20, params=prm,
                                          want_scores=True)
    J = slice(n_sink, N - n_recent)
    e = fused[0, 0, J]
    lower = maximum_filter1d(e, size=3, mode="nearest") > e
    assert lower.any() and (~lower).any()
    np.testing.assert_allclose(ref[0, 0, J] - e, np.where(lower, np.log(0.5), 0.0), atol=1e-12)


def test_cross_head_exclusivity_is_permutation_equivariant(orc):
    g = np.random.default_rng(9)
    N, Hkv, G = 400, 4, 2
    z = g.normal(size=(1, Hkv * G, N)) * 2
    kn = g.uniform(0.5, 2.0, size=(1, Hkv, N))
    idx, n_idx, _, ref = orc.select_refined([N], Hkv * G, Hkv, z, 4, 40, 25, key_norm=kn,
                                            want_scores=True)
    perm = [2, 0, 3, 1]
    zq = z.reshape(1, Hkv, G, N)[:, perm].reshape(1, Hkv * G, N)
    idx2, n2, _, ref2 = orc.select_refined([N], Hkv * G, Hkv, zq, 4, 40, 25,
                                           key_norm=kn[:, perm], want_scores=True)
    assert (idx2[0] == idx[0, perm]).all() and (n2[0] == n_idx[0, perm]).all()
    np.testing.assert_array_equal(ref2[0], ref[0, perm])
    # against the same pipeline without exclusivity: at every position the best head keeps
    # its score and every other head loses exactly log(1 - alpha_cross)
    _, _, _, nms = orc.select_refined([N], Hkv * G, Hkv, z, 4, 40, 25, key_norm=kn,
                                      params=dict(alpha_cross=0.0), want_scores=True)
    J = slice(4, N - 40)
    e, r = nms[0, :, J], ref[0, :, J]
    best = e == e.max(axis=0, keepdims=True)
    np.testing.assert_allclose(r - e, np.where(best, 0.0, np.log(0.65)), atol=1e-12)


# -------------------------------------------------------------------------------- mask

def test_sink_mask_library_sort(orc):
    g = torch.Generator().manual_seed(14)
    B, Hq = 3, 64
    z0 = torch.randn((B, Hq), generator=g).double()
    lse = z0 + torch.rand((B, Hq), generator=g).double() * 3
    # batch 2: only four distinct p0 values, so the cut falls inside a group of ties
    z0[2] = 0.0
    lse[2] = torch.randint(1, 5, (Hq,), generator=g).double() / 2
    for frac in (0.0, 0.25, 0.3, 0.5, 1.0):
        m = orc.sink_mask(z0, lse, frac)
        for b in range(B):
            p0 = np.exp((z0[b] - lse[b]).numpy())
            order = np.lexsort((np.arange(Hq), -p0))[:int(math.floor(frac * Hq))]
            exp = np.zeros(Hq, np.uint8)
            exp[order] = 1
            assert (m[b] == exp).all()
    with pytest.raises(ValueError):
        orc.sink_mask(z0, lse, 1.5)


# ------------------------------------------------------------------------- group routing

def _routed_case(orc, seed=15):
    wl = synth.Workload("route_tiny", 300 + seed, 3, 8, 2, 32, "bf16", 400, 4, 20, 60, 3,
                        sink=True)
    lay = synth.make_layer(wl, 0, lens=[400, 250, 0])
    q = synth.make_query(wl, 0, 1, u=lay.u, n_for_sink=400)
    lens = [401, 251, 0]
    idx, n_idx = synth.synthetic_index_set(lay, "scattered", seed=seed)
    c = orc.Cache(lay.k, lay.v, torch.tensor(lens, dtype=torch.int32), wl.Hq)
    return wl, lay, q, lens, idx, n_idx, c


def test_routed_decision_matches_dense_position0_logit(orc):
    """The routing decision equals the rule applied to the dense oracle's logit at position 0,
    for a normaliser chosen head by head to land well clear of the threshold."""
    wl, lay, q, lens, idx, n_idx, c = _routed_case(orc)
    _, _, z = orc.dense(c, q)
    g = torch.Generator().manual_seed(1)
    gamma = 0.65
    # each head's estimated token-0 mass is set to 0.9 (sink) or 0.3 (not) by its normaliser
    target = torch.where(torch.rand((wl.B, wl.Hq), generator=g) < 0.7, 0.9, 0.3).double()
    z0 = torch.tensor(np.nan_to_num(z[:, :, 0], nan=0.0))
    route_lse = z0 - torch.log(target)
    out, lse, routed, margin = orc.sparse_routed(c, q, idx, n_idx, wl.n_recent, route_lse, gamma)
    G = wl.G
    for b in range(wl.B):
        for h in range(wl.Hkv):
            heads = target[b, h * G:(h + 1) * G]
            expect = lens[b] > 0 and bool((heads >= gamma).all())
            assert routed[b, h] == expect
            if lens[b] > 0:
                assert abs(margin[b, h] - float(torch.log(heads / gamma).min())) < 1e-9
            if expect:
                assert (out[b, h * G:(h + 1) * G] == 0).all()
                assert np.isneginf(lse[b, h * G:(h + 1) * G]).all()


def test_routed_reduces_to_sparse_and_to_zeros(orc):
    wl, lay, q, lens, idx, n_idx, c = _routed_case(orc, seed=16)
    base_o, base_l = orc.sparse(c, q, idx, n_idx, wl.n_recent)
    # a normaliser far above every token-0 logit routes nothing: exactly the plain fast step
    hi = torch.full((wl.B, wl.Hq), 1e6, dtype=torch.float64)
    o, l, routed, _ = orc.sparse_routed(c, q, idx, n_idx, wl.n_recent, hi, 0.65)
    assert routed.sum() == 0
    assert np.array_equal(o, base_o) and np.array_equal(l, base_l)
    # far below: every group with history is bypassed, all its heads output exact zeros
    lo = torch.full((wl.B, wl.Hq), -1e6, dtype=torch.float64)
    o, l, routed, _ = orc.sparse_routed(c, q, idx, n_idx, wl.n_recent, lo, 0.65)
    assert routed.tolist() == [[1, 1], [1, 1], [0, 0]]           # len 0: nothing to route
    assert (o == 0).all() and np.isneginf(l[:2]).all()
    # a head mask still zeroes its heads in groups that are not routed
    hm = torch.zeros((wl.B, wl.Hq), dtype=torch.uint8)
    hm[0, 1] = 1
    o, _, _, _ = orc.sparse_routed(c, q, idx, n_idx, wl.n_recent, hi, 0.65, head_mask=hm)
    assert (o[0, 1] == 0).all()
    assert np.array_equal(o[0, 0], base_o[0, 0])
