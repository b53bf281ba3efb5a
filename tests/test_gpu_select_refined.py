"""The full Selector (sfi_select_refined) on the GPU against the fp64 oracle.

The refinements take discrete decisions (is a neighbour larger, is another head larger) on
scores that the GPU computes in fp32 and the oracle in fp64.  Where the oracle's decision
margin is below DELTA (natural-log units) either outcome is accepted for that position, as is
any position whose refined score lies within DELTA of the k-th largest; every other position
must agree.  Planted inputs keep those sets small or empty, and the tests check that the
refinements do change the selection there.
"""
import numpy as np
import pytest
import torch

from sparse_kv_attention_dense_amd import binding as B
from sparse_kv_attention_dense_amd import synth

from gpu_util import DEV, gpu_select, round4, say

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
DELTA = 5e-5
CHUNKED_MAX_LEN = 300000
PASSES_MAX_LEN = 1100000          # k_sel + max_len / 64 > 16384: no finish pass


def _gpu_refined(wl, lens, z, kn, params, n_sink, n_recent, k_sel, max_len=None, norm_pad=0):
    """norm_pad: extra floats per key-norm row (an odd number leaves the rows unaligned, so
    the norms are read one by one instead of in 16-byte loads)."""
    max_len = max_len or max(lens)
    stride = round4(max(max_len, z.shape[-1]))
    nstride = stride + norm_pad
    lens_dev = torch.tensor(lens, dtype=torch.int32, device=DEV)
    desc = B.KVDesc.for_logits(lens_dev, max_len, wl.Hq, wl.Hkv, wl.d)
    zd = torch.zeros((len(lens), wl.Hq, stride), device=DEV)
    zd[:, :, :z.shape[-1]] = z.to(DEV)
    knd = None
    if kn is not None:
        knd = torch.ones((len(lens), wl.Hkv, nstride), device=DEV)
        knd[:, :, :kn.shape[-1]] = kn.to(DEV)
    idx_stride = n_sink + k_sel
    idx = torch.full((len(lens), wl.Hkv, idx_stride), -7, dtype=torch.int32, device=DEV)
    n_idx = torch.full((len(lens), wl.Hkv), -7, dtype=torch.int32, device=DEV)
    ws = torch.zeros(B.sfi_workspace_bytes(desc, B.SFI_OP_SELECT_REFINED), dtype=torch.uint8,
                     device=DEV)
    B.sfi_select_refined(desc, zd, stride, knd, nstride, n_sink, n_recent, k_sel, params, idx,
                         idx_stride, n_idx, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), n_idx.cpu().numpy()


def _compare(orc, wl, lens, z, kn, params, n_sink, n_recent, k_sel, ig, ng):
    """GPU selection against the oracle's; returns (differing positions, ambiguous ones)."""
    zz = z.double().numpy()
    knn = None if kn is None else kn.double().numpy()
    eidx, en, fused, refined = orc.select_refined(lens, wl.Hq, wl.Hkv, zz, n_sink, n_recent,
                                                  k_sel, key_norm=knn, params=params,
                                                  want_scores=True)
    _, _, _, nms = orc.select_refined(lens, wl.Hq, wl.Hkv, zz, n_sink, n_recent, k_sel,
                                      key_norm=knn, params=dict(params, alpha_cross=0.0),
                                      want_scores=True)
    n_diff = n_amb = 0
    for b, N in enumerate(lens):
        J0, J1 = n_sink, N - n_recent
        for h in range(wl.Hkv):
            assert ng[b, h] == en[b, h], f"n_idx differs at ({b},{h})"
            g = ig[b, h, :ng[b, h]]
            o = eidx[b, h, :en[b, h]]
            assert (np.diff(g) > 0).all()
            ns = min(n_sink, N)
            assert (g[:ns] == np.arange(ns)).all()
            if J1 <= J0:
                assert np.array_equal(g, o)
                continue
            e = fused[b, h, J0:J1]
            amb = np.zeros(J1 - J0, bool)
            amb[1:] |= np.abs(e[1:] - e[:-1]) < DELTA            # Soft-NMS near-ties
            amb[:-1] |= np.abs(e[:-1] - e[1:]) < DELTA
            if wl.Hkv > 1:
                others = np.delete(nms[b, :, J0:J1], h, axis=0).max(axis=0)
                amb |= np.abs(nms[b, h, J0:J1] - others) < DELTA  # exclusivity near-ties
            rJ = refined[b, h, J0:J1]
            kth = np.sort(rJ)[::-1][min(k_sel, len(rJ)) - 1] if k_sel > 0 else np.inf
            amb |= np.abs(rJ - kth) < DELTA                       # Top-K boundary
            n_amb += int(amb.sum())
            if np.array_equal(g, o):
                continue
            diff = np.setxor1d(g, o)
            assert amb[diff - J0].all(), f"({b},{h}): sets differ at unambiguous positions"
            n_diff += len(diff)
    return n_diff, n_amb, eidx, en


def _position_norms(B_, Hkv, n, seed):
    """Key norms that depend on the position only (the same for every KV head)."""
    g = torch.Generator().manual_seed(seed)
    row = torch.rand(n, generator=g) * 1.5 + 0.5
    return row.repeat(B_, Hkv, 1)


@pytest.mark.parametrize("name,lens", [("gqa4_32k", [5003]), ("sink_128k_b4", [9001, 12345]),
                                       ("gqa8_512k", [40000])])
def test_refined_zero_parameters_is_the_plain_selector(orc, name, lens):
    wl = W[name]
    say(f"[refined 0] {name} lens={lens}")
    z, ranks = synth.planted_logits(len(lens), wl.Hq, wl.Hkv, lens, wl.n_sink, wl.n_recent,
                                    round4(max(lens)), seed=3, noise_sink=40.0)
    zero = dict(lambda_=0.0, alpha_soft=0.0, alpha_cross=0.0)
    ig, ng = _gpu_refined(wl, lens, z, None, zero, wl.n_sink, wl.n_recent, wl.k_sel,
                          max_len=CHUNKED_MAX_LEN)
    pi, pn = gpu_select(torch.tensor(lens, dtype=torch.int32, device=DEV), CHUNKED_MAX_LEN, wl,
                        _pad(z, CHUNKED_MAX_LEN), round4(CHUNKED_MAX_LEN))
    assert np.array_equal(ig, pi.cpu().numpy()) and np.array_equal(ng, pn.cpu().numpy())
    for b, N in enumerate(lens):
        for h in range(wl.Hkv):
            keep = sorted((torch.nonzero(ranks[b][h] < wl.k_sel).flatten() + wl.n_sink).tolist())
            assert ig[b, h, :ng[b, h]].tolist() == list(range(min(wl.n_sink, N))) + keep


def _pad(z, n):
    zd = torch.zeros((z.shape[0], z.shape[1], round4(n)), device=DEV)
    zd[:, :, :z.shape[-1]] = z.to(DEV)
    return zd


@pytest.mark.parametrize("name,lens,norms", [("gqa4_32k", [5003], "position"),
                                             ("sink_128k_b4", [9001, 12345], "position"),
                                             ("ragged_paged_b16", [2500, 4097, 8200], "random"),
                                             ("gqa8_512k", [40000], "none")])
def test_refined_planted(orc, name, lens, norms):
    wl = W[name]
    say(f"[refined planted] {name} lens={lens} norms={norms}")
    z, _ = synth.planted_logits(len(lens), wl.Hq, wl.Hkv, lens, wl.n_sink, wl.n_recent,
                                round4(max(lens)), seed=4, noise_sink=40.0)
    n = z.shape[-1]
    kn = None
    if norms == "position":
        kn = _position_norms(len(lens), wl.Hkv, n, seed=5)
    elif norms == "random":
        g = torch.Generator().manual_seed(6)
        kn = torch.rand((len(lens), wl.Hkv, n), generator=g) * 1.5 + 0.5
    params = dict(B.REFINE_DEFAULTS)
    ig, ng = _gpu_refined(wl, lens, z, kn, params, wl.n_sink, wl.n_recent, wl.k_sel,
                          max_len=CHUNKED_MAX_LEN)
    n_diff, n_amb, eidx, en = _compare(orc, wl, lens, z, kn, params, wl.n_sink, wl.n_recent,
                                       wl.k_sel, ig, ng)
    # the refinements matter on this input
    pidx, pn, _ = orc.select(lens, wl.Hq, wl.Hkv, z.double().numpy(), wl.n_sink, wl.n_recent,
                             wl.k_sel)
    changed = sum(len(np.setxor1d(pidx[b, h, :pn[b, h]], eidx[b, h, :en[b, h]]))
                  for b in range(len(lens)) for h in range(wl.Hkv))
    say(f"    positions changed by the refinements: {changed}; GPU vs oracle differ at {n_diff} "
        f"(ambiguous {n_amb})")
    assert changed > 0
    assert n_diff <= n_amb


def test_refined_unaligned_norm_rows():
    """Key-norm rows whose stride is not a multiple of 4 (read one by one) select exactly what
    aligned rows (read 16 bytes at a time) select."""
    wl = W["ragged_paged_b16"]
    lens = [2500, 4097, 8200]
    say(f"[refined unaligned norms] {wl.name} lens={lens}")
    z, _ = synth.planted_logits(len(lens), wl.Hq, wl.Hkv, lens, wl.n_sink, wl.n_recent,
                                round4(max(lens)), seed=10, noise_sink=40.0)
    g = torch.Generator().manual_seed(11)
    kn = torch.rand((len(lens), wl.Hkv, z.shape[-1]), generator=g) * 1.5 + 0.5
    params = dict(B.REFINE_DEFAULTS)
    ia, na = _gpu_refined(wl, lens, z, kn, params, wl.n_sink, wl.n_recent, wl.k_sel)
    for pad in (1, 3):
        ib, nb = _gpu_refined(wl, lens, z, kn, params, wl.n_sink, wl.n_recent, wl.k_sel,
                              norm_pad=pad)
        assert np.array_equal(ia, ib) and np.array_equal(na, nb), f"norm_pad={pad}"


def test_refined_on_dense_logits(orc):
    """Logits of a real slow step (the oracle's dense step on a sink workload, rounded to fp32)
    and the cache's key norms, fed to both sides."""
    wl = W["sink_128k_b4"].scaled(20011, B=2)
    say(f"[refined dense logits] {wl.name}")
    lay = synth.make_layer(wl, 0)
    q = synth.make_query(wl, 0, 0, u=lay.u)
    N = lay.len0_host
    _, _, logits = orc.dense(orc.Cache(lay.k, lay.v, torch.tensor(N, dtype=torch.int32), wl.Hq),
                             q)
    z = torch.from_numpy(logits[:, :, :max(N)]).float()
    kn = torch.stack([torch.stack([synth.logical_kv(lay, b, h, max(N))[0].norm(dim=-1)
                                   for h in range(wl.Hkv)]) for b in range(wl.B)])
    params = dict(B.REFINE_DEFAULTS)
    ig, ng = _gpu_refined(wl, N, z, kn, params, wl.n_sink, wl.n_recent, wl.k_sel)
    n_diff, n_amb, _, _ = _compare(orc, wl, N, z, kn, params, wl.n_sink, wl.n_recent,
                                   wl.k_sel, ig, ng)
    say(f"    GPU vs oracle differ at {n_diff} positions (ambiguous {n_amb})")
    assert n_diff <= n_amb


def test_refined_full_size(orc):
    wl = W["sink_128k_b4"]
    lens = synth.slow_step_lengths(wl)
    say(f"[refined planted full] {wl.name} B={wl.B} N={wl.n0} k={wl.k_sel}")
    z, _ = synth.planted_logits(len(lens), wl.Hq, wl.Hkv, lens, wl.n_sink, wl.n_recent,
                                round4(max(lens)), seed=7, noise_sink=40.0)
    kn = _position_norms(len(lens), wl.Hkv, z.shape[-1], seed=8)
    params = dict(B.REFINE_DEFAULTS)
    ig, ng = _gpu_refined(wl, lens, z, kn, params, wl.n_sink, wl.n_recent, wl.k_sel)
    n_diff, n_amb, _, _ = _compare(orc, wl, lens, z, kn, params, wl.n_sink, wl.n_recent,
                                   wl.k_sel, ig, ng)
    say(f"    GPU vs oracle differ at {n_diff} positions (ambiguous {n_amb})")
    assert n_diff <= n_amb


def test_refined_edges(orc):
    """Empty J, J shorter than k, k = 0, one KV head (no competition), no tail brake, no
    key norms, G = 1, and 20 KV heads (beyond the 8 the refine pass holds in registers at a
    time: three groups of heads, the scores computed twice)."""
    wl = synth.Workload("ref_edges", 1, 6, 6, 6, 64, "bf16", 3000, 4, 64, 100, 1)
    g = torch.Generator().manual_seed(9)
    lens = [3, 68, 150, 3000, 1, 2000]
    z = torch.randn((len(lens), wl.Hq, max(lens)), generator=g) * 3
    for params, k_sel in [(dict(B.REFINE_DEFAULTS), 100), (dict(B.REFINE_DEFAULTS, tail_frac=0.0), 0),
                          (dict(B.REFINE_DEFAULTS, alpha_cross=0.9, alpha_soft=0.0), 37)]:
        ig, ng = _gpu_refined(wl, lens, z, None, params, wl.n_sink, wl.n_recent, k_sel,
                              max_len=CHUNKED_MAX_LEN)
        n_diff, n_amb, _, _ = _compare(orc, wl, lens, z, None, params, wl.n_sink, wl.n_recent,
                                       k_sel, ig, ng)
        assert n_diff <= n_amb
        # a bound this long ends the chunked Selector in its resolve and emit passes instead of
        # the finish: the same keys, so the same indices
        ip, nq = _gpu_refined(wl, lens, z, None, params, wl.n_sink, wl.n_recent, k_sel,
                              max_len=PASSES_MAX_LEN)
        assert np.array_equal(ip, ig) and np.array_equal(nq, ng)
    # more KV heads than the exclusivity pass holds in registers
    many = synth.Workload("ref_many", 1, 2, 40, 20, 128, "bf16", 6000, 4, 64, 200, 1)
    zm = torch.randn((2, 40, 6000), generator=g) * 2
    km = torch.rand((2, 20, 6000), generator=g) + 0.5
    ig, ng = _gpu_refined(many, [6000, 5000], zm, km, dict(B.REFINE_DEFAULTS), 4, 64, 200)
    n_diff, n_amb, _, _ = _compare(orc, many, [6000, 5000], zm, km, dict(B.REFINE_DEFAULTS), 4,
                                   64, 200, ig, ng)
    assert n_diff <= n_amb
    one = synth.Workload("ref_one", 1, 2, 3, 1, 128, "bf16", 9000, 4, 64, 300, 1)
    z1 = torch.randn((2, 3, 9000), generator=g) * 2
    ig, ng = _gpu_refined(one, [9000, 7000], z1, None, dict(B.REFINE_DEFAULTS), 4, 64, 300)
    n_diff, n_amb, _, _ = _compare(orc, one, [9000, 7000], z1, None, dict(B.REFINE_DEFAULTS), 4,
                                   64, 300, ig, ng)
    assert n_diff <= n_amb
