"""Selector on the GPU against the fp64 oracle, fed the same fp32 logits buffer."""
import numpy as np
import pytest
import torch

from sparse_kv_attention_dense_amd import synth

from gpu_util import DEV, compare_index_sets, gpu_select, round4, say

pytestmark = pytest.mark.gpu


# The library runs the Selector either as one workgroup per (b, KV head) or as chunked
# kernels, choosing from the descriptor (unit logit bytes against all logit bytes).  A
# declared max_len far above the real lengths makes it choose the chunked kernels, so both
# paths run the same cases.
CHUNKED_MAX_LEN = 300000
# a declared bound this long makes the chunked Selector end in its resolve and emit passes
# instead of the one-workgroup-per-unit finish (k_sel + max_len / 64 > 16384 entries)
PASSES_MAX_LEN = 1100000
MAX_LEN_OF = {"unit": None, "chunked": CHUNKED_MAX_LEN, "chunked_passes": PASSES_MAX_LEN}


def _run(orc, wl, lens, z, exact, n_sink=None, n_recent=None, k_sel=None, idx_stride=None,
         max_len=None):
    n_sink = wl.n_sink if n_sink is None else n_sink
    n_recent = wl.n_recent if n_recent is None else n_recent
    k_sel = wl.k_sel if k_sel is None else k_sel
    idx_stride = idx_stride or (n_sink + k_sel)
    max_len = max_len or max(lens)
    stride = round4(max(max_len, z.shape[-1]))
    lens_dev = torch.tensor(lens, dtype=torch.int32, device=DEV)
    zd = torch.zeros((z.shape[0], z.shape[1], stride), device=DEV)
    zd[:, :, :z.shape[-1]] = z.to(DEV)
    idx, n_idx = gpu_select(lens_dev, max_len, wl, zd, stride, n_sink, n_recent, k_sel, idx_stride)
    eidx, en, f = orc.select(lens, wl.Hq, wl.Hkv, z, n_sink, n_recent, k_sel, idx_stride,
                             want_f=True)
    swaps = compare_index_sets(idx, n_idx, eidx, en, f, lens, n_sink, n_recent, k_sel, exact)
    return idx, n_idx, swaps


def _planted(wl, lens, seed, noise=40.0, n_sink=None, n_recent=None):
    n_sink = wl.n_sink if n_sink is None else n_sink
    n_recent = wl.n_recent if n_recent is None else n_recent
    z, ranks = synth.planted_logits(len(lens), wl.Hq, wl.Hkv, lens, n_sink, n_recent,
                                    round4(max(lens)), seed, noise_sink=noise)
    return z, ranks


W = synth.WORKLOADS


@pytest.mark.parametrize("name,lens", [("gqa4_32k", [5003]), ("sink_128k_b4", [9001, 12345]),
                                       ("ragged_paged_b16", [2500, 3333, 4097, 8200]),
                                       ("gqa8_512k", [40000]), ("tiny_2k_f32", [2048])])
def test_select_planted_is_exact(orc, name, lens):
    wl = W[name]
    say(f"[select planted] {name} lens={lens}")
    z, ranks = _planted(wl, lens, seed=sum(map(ord, name)))
    idx, n_idx, _ = _run(orc, wl, lens, z, exact=True)
    # and the planted expectation itself
    ig = idx.cpu().numpy()
    for b, N in enumerate(lens):
        for h in range(wl.Hkv):
            keep = sorted((torch.nonzero(ranks[b][h] < wl.k_sel).flatten() + wl.n_sink).tolist())
            assert ig[b, h, :n_idx[b, h]].tolist() == list(range(min(wl.n_sink, N))) + keep


@pytest.mark.parametrize("name", ["sink_128k_b4", "gqa8_512k", "ragged_paged_b16", "gqa4_32k"])
def test_select_planted_full_size(orc, name):
    wl = W[name]
    lens = synth.slow_step_lengths(wl)
    say(f"[select planted full] {name} B={wl.B} N={wl.n0} k={wl.k_sel}")
    z, _ = _planted(wl, lens, seed=17)
    _run(orc, wl, lens, z, exact=True)


@pytest.mark.parametrize("seed,path", [(1, "unit"), (2, "unit"), (3, "chunked")])
def test_select_random_logits_band(orc, seed, path):
    wl = W["ragged_paged_b16"]
    # lengths short enough that one workgroup per unit is estimated faster, or long ones
    # declared with a far larger max_len for the chunked kernels
    lens = [2048, 2500, 3000, 1500] if path == "unit" else [8192, 9000, 20000, 32768]
    g = torch.Generator().manual_seed(seed)
    z = (torch.randn((4, wl.Hq, max(lens)), generator=g) * 2.0)
    _, _, swaps = _run(orc, wl, lens, z, exact=False,
                       max_len=CHUNKED_MAX_LEN if path == "chunked" else None)
    say(f"    tie-band swaps: {swaps}")


@pytest.mark.parametrize("path", ["unit", "chunked", "chunked_passes"])
def test_select_edges(orc, path):
    wl = synth.Workload("sel_edges", 1, 6, 8, 2, 128, "bf16", 5000, 4, 64, 100, 1)
    g = torch.Generator().manual_seed(3)
    ml = MAX_LEN_OF[path]
    say(f"[select edges] {path}")
    # |J| = 0 (N - n_r <= n_s), N < n_s, |J| < k_sel (take all), |J| = k_sel, chunk edges
    lens = [60, 2, 150, 168, 4096 + 68, 8192 + 69]
    z = torch.randn((6, 8, round4(max(lens))), generator=g)
    _run(orc, wl, lens, z, exact=True, max_len=ml)
    # k_sel = 0 keeps only sinks; n_sink = 0 keeps no sinks; an odd n_sink starts J mid-quad
    _run(orc, wl, lens, z, exact=True, k_sel=0, idx_stride=8, max_len=ml)
    _run(orc, wl, lens, z, exact=True, n_sink=0, k_sel=37, max_len=ml)
    _run(orc, wl, lens, z, exact=True, n_sink=3, n_recent=5, k_sel=101, max_len=ml)
    # no recent window: J runs to the end of the sequence
    _run(orc, wl, lens, z, exact=True, n_recent=0, k_sel=90, max_len=ml)
    # many exact ties: quantised logits, lowest positions win
    zq = torch.randint(-2, 2, z.shape, generator=g).float()
    _run(orc, wl, lens, zq, exact=True, max_len=ml)
    _run(orc, wl, lens, zq, exact=True, k_sel=1, idx_stride=5, max_len=ml)
    # every key equal: the first k_sel positions of J
    _run(orc, wl, lens, torch.zeros_like(z), exact=True, max_len=ml)


@pytest.mark.parametrize("case", range(12))
def test_select_chunked_random_shapes(orc, case):
    """Seeded random shapes for the chunked Selector, planted ranks (one exact answer): batch
    1-4, 1-8 KV heads, groups of 1-8 query heads, ragged lengths up to 40000, 0-8 sinks, a
    recent window of 0-300 and a budget from 0 to past |J|.  Both endings of the chunked path
    (the finish, and the resolve and emit passes) against the oracle and the planted set, and
    against each other bit for bit."""
    rng = np.random.default_rng(1000 + case)
    Bn = int(rng.integers(1, 5))
    Hkv = int(rng.integers(1, 9))
    G = int(rng.choice([1, 2, 4, 8]))
    lens = [int(x) for x in rng.integers(1, 40001, size=Bn)]
    n_sink = int(rng.integers(0, 9))
    n_recent = int(rng.integers(0, 301))
    nJ = max(0, max(lens) - n_sink - n_recent)
    k_sel = int(rng.integers(0, max(2, min(nJ + 50, 6000))))
    wl = synth.Workload(f"sel_rand{case}", 1, Bn, Hkv * G, Hkv, 128, "bf16", max(lens), n_sink,
                        n_recent, k_sel, 1)
    say(f"[select random shape {case}] B={Bn} Hkv={Hkv} G={G} lens={lens} sink={n_sink} "
        f"recent={n_recent} k={k_sel}")
    z, ranks = _planted(wl, lens, seed=77 + case, n_sink=n_sink, n_recent=n_recent)
    # 40000 positions with k <= 6000: the finish; 1100000: the resolve and emit passes
    istride = max(1, n_sink + k_sel)
    a = _run(orc, wl, lens, z, exact=True, n_sink=n_sink, n_recent=n_recent, k_sel=k_sel,
             idx_stride=istride, max_len=40000)
    b = _run(orc, wl, lens, z, exact=True, n_sink=n_sink, n_recent=n_recent, k_sel=k_sel,
             idx_stride=istride, max_len=PASSES_MAX_LEN)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    ig, ng = a[0].cpu().numpy(), a[1].cpu().numpy()
    for bi, N in enumerate(lens):
        for h in range(Hkv):
            keep = sorted((torch.nonzero(ranks[bi][h] < k_sel).flatten() + n_sink).tolist())
            assert ig[bi, h, :ng[bi, h]].tolist() == list(range(min(n_sink, N))) + keep


def test_select_finish_beyond_its_lds(orc):
    """The finish holds 16384 entries (kept keys and candidates of a unit) in LDS and reads the
    rest where the candidate pass wrote them: all keys equal (every key of J is an entry: 20000
    entries in the longer unit, 8932 in the shorter) and quantised logits with mass ties, against
    the oracle exactly, and bit for bit against the resolve and emit passes."""
    wl = synth.Workload("sel_fin", 1, 2, 8, 2, 128, "bf16", 20068, 4, 64, 100, 1)
    g = torch.Generator().manual_seed(11)
    lens = [20068, 9000]
    # a bound of 40000 positions keeps the chunked path with the finish for k_sel <= 15759
    for z in (torch.zeros((2, 8, 20068)),
              torch.randint(-1, 2, (2, 8, 20068), generator=g).float()):
        for k_sel in (100, 5000):
            say(f"[select finish overflow] k_sel={k_sel}")
            a = _run(orc, wl, lens, z, exact=True, k_sel=k_sel, max_len=40000)
            b = _run(orc, wl, lens, z, exact=True, k_sel=k_sel, max_len=PASSES_MAX_LEN)
            assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("path", ["unit", "chunked"])
def test_select_observation_window(orc, path):
    """Evidence over an observation window of W = 16 queries per head: the window's logits as
    rows i*W + w, 64 rows per KV head at G = 4, planted (exact) and random (tie band); and
    every head's row repeated W times selects what the row alone selects."""
    G, Hkv, Wn = 4, 2, 16
    wl = synth.Workload("sel_window", 1, 2, G * Hkv * Wn, Hkv, 128, "bf16", 20000, 4, 256, 300, 1)
    lens = [1000, 900] if path == "unit" else [20000, 15000]
    ml = CHUNKED_MAX_LEN if path == "chunked" else None
    say(f"[select window] {path} rows per KV head {G * Wn}")
    z, _ = _planted(wl, lens, seed=91)
    _run(orc, wl, lens, z, exact=True, max_len=ml)
    g = torch.Generator().manual_seed(92)
    _run(orc, wl, lens, torch.randn((2, wl.Hq, max(lens)), generator=g) * 2.0, exact=False,
         max_len=ml)
    one = synth.Workload("sel_window_1", 1, 2, G * Hkv, Hkv, 128, "bf16", 20000, 4, 256, 300, 1)
    z1, ranks = _planted(one, lens, seed=93)
    idx, n_idx, _ = _run(orc, wl, lens, z1.repeat_interleave(Wn, dim=1), exact=True, max_len=ml)
    ig = idx.cpu().numpy()
    for b, N in enumerate(lens):
        for h in range(Hkv):
            keep = sorted((torch.nonzero(ranks[b][h] < one.k_sel).flatten() + one.n_sink).tolist())
            assert ig[b, h, :n_idx[b, h]].tolist() == list(range(min(one.n_sink, N))) + keep


@pytest.mark.parametrize("G,path", [(1, "unit"), (16, "unit"), (1, "chunked"), (16, "chunked"),
                                    (5, "unit")])
def test_select_group_sizes(orc, G, path):
    wl = synth.Workload(f"sel_G{G}", 1, 2, 2 * G, 2, 128, "bf16", 20000, 4, 256, 700, 1)
    # short enough that one workgroup per unit is the estimated-faster path at every G
    lens = [3000, 2500] if path == "unit" else [20000, 15000]
    z, _ = _planted(wl, lens, seed=G)
    _run(orc, wl, lens, z, exact=True, max_len=CHUNKED_MAX_LEN if path == "chunked" else None)


def test_select_beyond_one_chunk_group(orc):
    """A context of more than 1024 Selector chunks (4M positions): the resolve pass then scans
    the per-chunk candidate numbers group by group.  Random logits, then all keys equal (every
    key is a candidate, more than fit in LDS)."""
    wl = synth.Workload("sel_4m", 1, 1, 2, 1, 128, "bf16", 4096 * 1024 + 5000, 4, 64, 2048, 1)
    lens = [4096 * 1024 + 5000]
    g = torch.Generator().manual_seed(11)
    z = torch.randn((1, 2, round4(lens[0])), generator=g)
    say("[select] 4M positions, random logits")
    _run(orc, wl, lens, z, exact=True, max_len=lens[0])
    say("[select] 4M positions, all keys equal")
    _run(orc, wl, lens, torch.zeros_like(z), exact=True, max_len=lens[0])


def test_select_deterministic():
    wl = W["sink_128k_b4"]
    lens = [30000, 20000]
    g = torch.Generator().manual_seed(9)
    z = torch.randn((2, wl.Hq, 30000), generator=g).to(DEV)
    lens_dev = torch.tensor(lens, dtype=torch.int32, device=DEV)
    a = gpu_select(lens_dev, 30000, wl, z, 30000)
    b = gpu_select(lens_dev, 30000, wl, z, 30000)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
