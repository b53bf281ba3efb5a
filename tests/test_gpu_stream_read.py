"""The measurement yardsticks: the streaming read (sfi_stream_read) reads every 16-byte word of
its buffer, the gather read (sfi_gather_read) the fast step's rows, and the group dot products
(sfi_group_dot) sum q_g . k_j over every row and head on both arithmetic units.

Its only visible effect is the sink word it writes when a thread's XOR of the words it read
equals the fixed constant.  Over a zeroed buffer with the constant planted in one word, the
thread that reads that word (and only it) sees the constant, so exactly one sink word, the one
of the workgroup whose chunk holds the planted word, must change: this checks the chunking,
the tail of a ragged last chunk and idle workgroups past the end.
"""
import pytest
import torch

from sparse_kv_attention_dense_amd import binding as B

from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9 - (1 << 32)          # the kernel's constant as an int32


@pytest.mark.parametrize("nbytes,wg", [(1 << 24, 1024), ((1 << 24) + 48, 1000), (4096, 4096)])
def test_stream_read_reads_every_word(nbytes, wg):
    say(f"[stream_read] bytes={nbytes} workgroups={wg}")
    n16 = nbytes // 16
    per = -(-n16 // wg)
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
    sink = torch.zeros(64, dtype=torch.int32, device=DEV)
    for k16 in sorted({0, 1, n16 // 2, per - 1, min(per, n16 - 1), 12345 % n16, n16 - 1}):
        word = 4 * k16 + k16 % 4
        buf.zero_()
        buf[word] = MAGIC
        sink.zero_()
        B.sfi_stream_read(buf, wg, sink)
        torch.cuda.synchronize()
        expect = torch.zeros_like(sink)
        expect[(k16 // per) % 64] = MAGIC
        assert torch.equal(sink, expect), f"planted word {word}"
    # a zeroed buffer leaves the sink alone
    buf.zero_()
    sink.fill_(5)
    B.sfi_stream_read(buf, wg, sink)
    torch.cuda.synchronize()
    assert torch.equal(sink, torch.full_like(sink, 5))


@pytest.mark.parametrize("paged", [False, True])
def test_gather_read_reads_the_fast_steps_rows(paged):
    """The gather yardstick (sfi_gather_read) reads the rows of the selected positions and of
    the recent window, and no other: over a zeroed cache with the kernel's constant planted in
    one key row, a sink word changes exactly when that row is one the fast step attends."""
    Bsz, Hkv, Hq, d, N, n_recent, bs = 2, 2, 8, 128, 3000, 64, 16
    g = torch.Generator().manual_seed(5)
    sel = [[sorted(torch.randperm(N - n_recent, generator=g)[:100].tolist()) for _ in range(Hkv)]
           for _ in range(Bsz)]
    idx = torch.zeros((Bsz, Hkv, 100), dtype=torch.int32)
    for b in range(Bsz):
        for h in range(Hkv):
            idx[b, h] = torch.tensor(sel[b][h], dtype=torch.int32)
    idx = idx.to(DEV)
    n_idx = torch.full((Bsz, Hkv), 100, dtype=torch.int32, device=DEV)
    lens = torch.full((Bsz,), N, dtype=torch.int32, device=DEV)
    nblk = (N + bs - 1) // bs
    if paged:
        perm = torch.randperm(Bsz * nblk, generator=g).to(torch.int32)
        bt = perm.view(Bsz, nblk).to(DEV)
        K = torch.zeros((Bsz * nblk, Hkv, bs, d), dtype=torch.bfloat16, device=DEV)
        desc = B.KVDesc(K, torch.zeros_like(K), lens, N, Hq, block_table=bt, block_size=bs)
    else:
        K = torch.zeros((Bsz, Hkv, N, d), dtype=torch.bfloat16, device=DEV)
        desc = B.KVDesc(K, torch.zeros_like(K), lens, N, Hq)
    words = K.view(torch.int32)                      # two bf16 per word, 64 words per row

    def row_words(b, h, pos):
        if paged:
            return words[int(bt[b, pos // bs]), h, pos % bs]
        return words[b, h, pos]

    sink = torch.zeros(64, dtype=torch.int32, device=DEV)
    cases = []
    for b in range(Bsz):
        for h in range(Hkv):
            s_set = set(sel[b][h])
            cases.append((b, h, sel[b][h][37], True))                       # selected
            cases.append((b, h, next(p for p in range(5, N) if p not in s_set and p < N - n_recent),
                          False))                                          # not selected
            cases.append((b, h, N - 5, True))                               # recent window
    for b, h, pos, hit in cases:
        K.zero_()
        row_words(b, h, pos)[3] = MAGIC
        sink.zero_()
        B.sfi_gather_read(desc, idx, 100, n_idx, n_recent, 64, sink)
        torch.cuda.synchronize()
        changed = bool((sink != 0).any())
        assert changed == hit, f"position {pos} of ({b},{h}): read {changed}, expected {hit}"
    say(f"    {len(cases)} planted rows: read exactly the fast step's rows")


def test_gather_read_split_past_one_table():
    """One workgroup per unit reading 5000 selected rows and the recent window: its slots
    span two row tables of 4096, and a planted row in the second table, in the recent window,
    and a row that is not selected are read, read, and not read."""
    Bsz, Hkv, Hq, d, N, n_recent, n_sel = 1, 2, 8, 128, 12000, 64, 5000
    g = torch.Generator().manual_seed(6)
    sel = [sorted(torch.randperm(N - n_recent, generator=g)[:n_sel].tolist()) for _ in range(Hkv)]
    idx = torch.tensor([sel], dtype=torch.int32).to(DEV)
    n_idx = torch.full((Bsz, Hkv), n_sel, dtype=torch.int32, device=DEV)
    lens = torch.full((Bsz,), N, dtype=torch.int32, device=DEV)
    K = torch.zeros((Bsz, Hkv, N, d), dtype=torch.bfloat16, device=DEV)
    desc = B.KVDesc(K, torch.zeros_like(K), lens, N, Hq)
    words = K.view(torch.int32)
    sink = torch.zeros(64, dtype=torch.int32, device=DEV)
    for h in range(Hkv):
        s_set = set(sel[h])
        cases = [(sel[h][4500], True),                                       # second table
                 (N - 3, True),                                              # recent window
                 (next(p for p in range(N - n_recent) if p not in s_set), False)]
        for pos, hit in cases:
            K.zero_()
            words[0, h, pos][5] = MAGIC
            sink.zero_()
            B.sfi_gather_read(desc, idx, n_sel, n_idx, n_recent, 1, sink)
            torch.cuda.synchronize()
            changed = bool((sink != 0).any())
            assert changed == hit, f"position {pos} of head {h}: read {changed}, expected {hit}"
    say("    rows past the first 4096-slot table read once each")


def _dot_case(n_rows, G, positive, seed):
    g = torch.Generator().manual_seed(seed)
    if positive:                        # every product positive: no cancellation in the sums
        rows = (0.5 + 1.5 * torch.rand(n_rows, 128, generator=g)).to(torch.bfloat16)
        q = (0.5 + 1.5 * torch.rand(G, 128, generator=g)).to(torch.bfloat16)
    else:
        rows = torch.randn(n_rows, 128, generator=g).to(torch.bfloat16)
        q = torch.randn(G, 128, generator=g).to(torch.bfloat16)
    dots = rows.double() @ q.double().T                  # [n_rows][G], exact in fp64
    return rows, q, float(dots.sum()), float(dots.abs().sum())


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("n_rows,wg", [(16 * 4099, 1024), (16 * 4099, 37), (16, 3)])
def test_group_dot_sums_every_product(G, n_rows, wg):
    """Units 1 (vector ALUs) and 2 (MFMA) against the fp64 sum of q_g . k_j over all rows and
    heads.  With positive inputs one missed 16-row group or head moves the sum by more than
    1/4100 of it, far above fp32 rounding (bound 2e-5 of the sum); with signed inputs the bound
    is 2e-5 of the sum of magnitudes.  Unit 0 leaves part alone.  Ragged: 4099 groups over 1024
    or 37 workgroups, and one group over 3 (two idle workgroups write zero)."""
    for positive in (True, False):
        say(f"[group_dot] G={G} rows={n_rows} wg={wg} positive={positive}")
        rows, q, ref, mag = _dot_case(n_rows, G, positive, seed=G * 1000 + n_rows % 997 + wg)
        rd, qd = rows.to(DEV), q.to(DEV)
        sink = torch.zeros(64, dtype=torch.int32, device=DEV)
        got = {}
        for unit in ("valu", "mfma"):
            part = torch.full((wg,), float("nan"), device=DEV)
            B.sfi_group_dot(rd, qd, unit, wg, part, sink)
            torch.cuda.synchronize()
            assert torch.isfinite(part).all(), unit
            got[unit] = float(part.double().sum())
            bound = 2e-5 * (abs(ref) if positive else mag)
            assert abs(got[unit] - ref) <= bound, (unit, got[unit], ref, bound)
        assert abs(got["valu"] - got["mfma"]) <= 2e-5 * mag
        part = torch.full((wg,), 7.0, device=DEV)
        B.sfi_group_dot(rd, qd, "read", wg, part, sink)
        torch.cuda.synchronize()
        assert bool((part == 7.0).all())
