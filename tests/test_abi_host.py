"""Host-only checks of libsfi.so: it loads, exports every function include/sfi.h declares,
and rejects bad arguments with the documented status before any GPU work is queued.
No test here needs a GPU (no call below passes validation)."""
import ctypes
import os
import re

import pytest

from sparse_kv_attention_dense_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # an aligned address that host code never dereferences


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B._LIB_PATH):
        from sparse_kv_attention_dense_amd import build
        build.build()
    return B.lib()


def _declared():
    text = open(os.path.join(ROOT, "include", "sfi.h")).read()
    return sorted(set(re.findall(r"\b(sfi_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = _declared()
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def _desc(**kw):
    d = B.sfi_kv_desc()
    d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim = 2, 32, 8, 128
    d.dtype = B.SFI_BF16
    d.k = d.v = FAKE
    d.n_cap = 4096
    d.block_table = None
    d.block_size = 0
    d.max_blocks = 0
    d.len = FAKE
    d.max_len = 4000
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _dense(L, d, ws_bytes=0, q=FAKE, out=FAKE, logits=FAKE, stride=4000):
    return L.sfi_dense_decode(ctypes.byref(d) if d is not None else None, q, out, FAKE, logits,
                              stride, FAKE if ws_bytes else None, ws_bytes, None)


def test_descriptor_validation(L):
    big = 1 << 40
    assert _dense(L, None, big) == B.SFI_E_INVALID
    assert _dense(L, _desc(num_q_heads=30), big) == B.SFI_E_INVALID          # G not an integer
    assert _dense(L, _desc(num_q_heads=8 * 17), big) == B.SFI_E_UNSUPPORTED  # G = 17
    assert _dense(L, _desc(head_dim=96), big) == B.SFI_E_UNSUPPORTED
    assert _dense(L, _desc(dtype=7), big) == B.SFI_E_UNSUPPORTED
    assert _dense(L, _desc(k=None), big) == B.SFI_E_INVALID
    assert _dense(L, _desc(k=FAKE + 4), big) == B.SFI_E_INVALID               # misaligned
    assert _dense(L, _desc(len=None), big) == B.SFI_E_INVALID
    assert _dense(L, _desc(n_cap=100), big) == B.SFI_E_INVALID                # max_len > n_cap
    assert _dense(L, _desc(block_table=FAKE, block_size=12, max_blocks=400), big) == B.SFI_E_INVALID
    assert _dense(L, _desc(block_table=FAKE, block_size=16, max_blocks=10), big) == B.SFI_E_INVALID
    assert _dense(L, _desc(), big, q=None) == B.SFI_E_INVALID
    assert _dense(L, _desc(), big, stride=3999) == B.SFI_E_INVALID            # stride < max_len
    assert _dense(L, _desc(), big, stride=4002) == B.SFI_E_INVALID            # stride % 4
    assert _dense(L, _desc(), 0) == B.SFI_E_WORKSPACE


def test_workspace_size_is_checked(L):
    d = _desc()
    need = L.sfi_workspace_bytes(ctypes.byref(d), B.SFI_OP_DENSE, 0, 0)
    assert need > 0
    assert _dense(L, d, need - 1) == B.SFI_E_WORKSPACE
    # misaligned workspace
    rc = L.sfi_dense_decode(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 4000, FAKE + 64, need, None)
    assert rc == B.SFI_E_WORKSPACE
    sp = L.sfi_workspace_bytes(ctypes.byref(d), B.SFI_OP_SPARSE, 4 + 2048, 256)
    assert sp > 0
    rc = L.sfi_sparse_decode(ctypes.byref(d), FAKE, FAKE, 2052, FAKE, 256, None, FAKE, FAKE,
                             FAKE, sp - 256, None)
    assert rc == B.SFI_E_WORKSPACE
    assert L.sfi_workspace_bytes(ctypes.byref(d), 9, 0, 0) == 0
    assert L.sfi_workspace_bytes(None, B.SFI_OP_DENSE, 0, 0) == 0


def test_select_and_mask_validation(L):
    d = _desc(k=None, v=None)
    ws = L.sfi_workspace_bytes(ctypes.byref(d), B.SFI_OP_SELECT, 0, 0)
    assert ws > 0
    sel = lambda **k: L.sfi_select(ctypes.byref(d), k.get("logits", FAKE), k.get("stride", 4000),
                                   k.get("ns", 4), k.get("nr", 256), k.get("ks", 2048),
                                   FAKE, k.get("istride", 2052), FAKE,
                                   FAKE, k.get("ws", ws - 1), None)
    assert sel() == B.SFI_E_WORKSPACE
    assert sel(istride=2051, ws=ws) == B.SFI_E_INVALID       # idx_stride < n_sink + k_sel
    assert sel(ks=-1, ws=ws) == B.SFI_E_INVALID
    assert sel(logits=None, ws=ws) == B.SFI_E_INVALID
    assert sel(stride=10, ws=ws) == B.SFI_E_INVALID
    assert sel(stride=4002, ws=ws) == B.SFI_E_INVALID          # stride not a multiple of 4
    assert sel(logits=FAKE + 4, ws=ws) == B.SFI_E_INVALID      # logits not 16-byte aligned
    mask = lambda frac, dd=d: L.sfi_sink_bypass_mask(ctypes.byref(dd), FAKE, 4000, FAKE,
                                                     ctypes.c_float(frac), None, None)
    assert mask(0.25) == B.SFI_E_INVALID                      # head_mask NULL
    ok_ptr = lambda frac: L.sfi_sink_bypass_mask(ctypes.byref(d), FAKE, 4000, FAKE,
                                                 ctypes.c_float(frac), FAKE + 1, None)
    assert ok_ptr(1.5) == B.SFI_E_INVALID
    assert ok_ptr(float("nan")) == B.SFI_E_INVALID
    assert ok_ptr(-0.1) == B.SFI_E_INVALID


def test_group_size_limits(L):
    """The attention calls hold a KV group in one 16-wide MFMA dimension; the Selector and the
    mask read logit rows only and take up to 64 per KV head (query heads x window queries)."""
    big = 1 << 40
    for G, sel_ok in ((16, True), (64, True), (65, False)):
        d = _desc(k=None, v=None, num_q_heads=2 * G, num_kv_heads=2)
        st = L.sfi_select(ctypes.byref(d), FAKE, 4000, 4, 256, 2048, FAKE, 2052, FAKE, FAKE, 0,
                          None)
        assert st == (B.SFI_E_WORKSPACE if sel_ok else B.SFI_E_UNSUPPORTED), G
        assert (L.sfi_workspace_bytes(ctypes.byref(d), B.SFI_OP_SELECT, 0, 0) > 0) == sel_ok
    d = _desc(num_q_heads=64, num_kv_heads=2)                      # G = 32
    assert _dense(L, d, big) == B.SFI_E_UNSUPPORTED
    assert L.sfi_workspace_bytes(ctypes.byref(d), B.SFI_OP_DENSE, 0, 0) == 0


def test_single_unit_paged_dense_up_to_the_table_capacity(L):
    """One (sequence, KV head) unit on a paged cache: splits grow up to the row table's 4096
    positions, so contexts up to 1024 x 4096 positions are planned; one more is rejected."""
    def desc(n):
        return _desc(batch=1, num_q_heads=2, num_kv_heads=1, head_dim=64, n_cap=0, max_len=n,
                     block_table=FAKE, block_size=16, max_blocks=(n + 15) // 16)
    for n in (2_200_000, 3_000_000, 1024 * 4096):
        assert L.sfi_workspace_bytes(ctypes.byref(desc(n)), B.SFI_OP_DENSE, 0, 0) > 0, n
    assert L.sfi_workspace_bytes(ctypes.byref(desc(1024 * 4096 + 1)), B.SFI_OP_DENSE, 0, 0) == 0


def test_sparse_validation(L):
    d = _desc()
    ws = L.sfi_workspace_bytes(ctypes.byref(d), B.SFI_OP_SPARSE, 2052, 256)
    sp = lambda **k: L.sfi_sparse_decode(ctypes.byref(d), FAKE, k.get("idx", FAKE),
                                         k.get("istride", 2052), FAKE, k.get("nr", 256), None,
                                         FAKE, None, FAKE, ws, None)
    assert sp(idx=None) == B.SFI_E_INVALID
    assert sp(istride=0) == B.SFI_E_INVALID
    assert sp(nr=-1) == B.SFI_E_INVALID
    # far more slots than one launch plans for
    assert L.sfi_workspace_bytes(ctypes.byref(d), B.SFI_OP_SPARSE, 1 << 30, 0) == 0


def test_noalloc_fast_step_validation(L):
    """The fast step on the library's static scratch array validates like sfi_sparse_decode and
    rejects, before any HIP call, a step whose partial records would not fit the array."""
    na = lambda dd, **k: L.sfi_sparse_decode_noalloc(ctypes.byref(dd), FAKE, k.get("idx", FAKE),
                                                     k.get("istride", 2052), FAKE,
                                                     k.get("nr", 256), None, FAKE, None, None)
    d = _desc()
    assert L.sfi_workspace_bytes(ctypes.byref(d), B.SFI_OP_SPARSE, 2052, 256) <= \
        B.SFI_NOALLOC_SCRATCH_BYTES
    assert na(d, idx=None) == B.SFI_E_INVALID
    assert na(d, istride=0) == B.SFI_E_INVALID
    assert na(d, nr=-1) == B.SFI_E_INVALID
    assert na(_desc(head_dim=96)) == B.SFI_E_UNSUPPORTED
    big = _desc(batch=4096, n_cap=4096)                 # 32768 units: records far past 8 MiB
    need = L.sfi_workspace_bytes(ctypes.byref(big), B.SFI_OP_SPARSE, 2052, 256)
    assert need > B.SFI_NOALLOC_SCRATCH_BYTES
    assert na(big) == B.SFI_E_SCRATCH


def test_step_descriptor_validation(L):
    """sfi_sparse_decode_step validates the host side (shapes, capacities, bounds, workspace)
    before any HIP call; the descriptor's own pointers are device data."""
    d = _desc(k=None, v=None, len=None, max_len=10 ** 9)    # pointers and max_len are not read
    ws = L.sfi_workspace_bytes(ctypes.byref(_desc()), B.SFI_OP_SPARSE, 2052, 256)
    st = lambda dd=d, step=FAKE, istride=2052, nr=256, w=ws: L.sfi_sparse_decode_step(
        ctypes.byref(dd) if dd is not None else None, step, istride, nr, FAKE if w else None, w,
        None)
    assert st(dd=None) == B.SFI_E_INVALID
    assert st(step=None) == B.SFI_E_INVALID
    assert st(step=FAKE + 4) == B.SFI_E_INVALID             # not 8-byte aligned
    assert st(istride=0) == B.SFI_E_INVALID
    assert st(nr=-1) == B.SFI_E_INVALID
    assert st(w=ws - 256) == B.SFI_E_WORKSPACE
    assert st(dd=_desc(head_dim=96)) == B.SFI_E_UNSUPPORTED
    assert ctypes.sizeof(B.sfi_step) == 12 * 8 + 8


def test_status_strings(L):
    for s in (B.SFI_OK, B.SFI_E_INVALID, B.SFI_E_UNSUPPORTED, B.SFI_E_WORKSPACE, B.SFI_E_HIP,
              B.SFI_E_SCRATCH):
        assert B.sfi_status_string(s).startswith("SFI_")
    assert "unknown" in B.sfi_status_string(42)


def test_workspace_grows_with_context(L):
    small = L.sfi_workspace_bytes(ctypes.byref(_desc(max_len=1000, n_cap=1000)), B.SFI_OP_SELECT, 0, 0)
    large = L.sfi_workspace_bytes(ctypes.byref(_desc(max_len=100000, n_cap=100000)), B.SFI_OP_SELECT, 0, 0)
    assert large > small > 0


def test_workspace_never_shrinks_as_length_grows(L):
    """A workspace sized for the longest step of a cycle must serve every shorter step."""
    for op, istride, nrec in ((B.SFI_OP_DENSE, 0, 0), (B.SFI_OP_SELECT, 0, 0),
                              (B.SFI_OP_SPARSE, 2052, 256)):
        for paged in (False, True):
            prev = 0
            for n in list(range(1, 600, 7)) + list(range(30000, 36000, 97)) + [131072, 524288 + 31]:
                kw = dict(max_len=n, n_cap=n, batch=1, num_q_heads=32, num_kv_heads=8)
                if paged:
                    kw.update(block_table=FAKE, block_size=16, max_blocks=(n + 15) // 16)
                need = L.sfi_workspace_bytes(ctypes.byref(_desc(**kw)), op, istride, nrec)
                assert need >= prev > 0 or (prev == 0 and need > 0), (op, paged, n, need, prev)
                prev = need


def test_slow_step_layers_validation(L):
    """Every layer is validated before anything is queued; the fake pointers below are never
    dereferenced because each call fails validation."""
    n = 3
    descs = (B.sfi_kv_desc * n)(*[_desc() for _ in range(n)])
    ptrs = lambda k, v=FAKE: (ctypes.c_void_p * k)(*([v] * k))
    # SFI_OP_SLOW bytes suffice for the dense workspace and for each Selector slot
    dws = sws = L.sfi_workspace_bytes(ctypes.byref(descs[0]), B.SFI_OP_SLOW, 0, 0)
    assert dws >= L.sfi_workspace_bytes(ctypes.byref(descs[0]), B.SFI_OP_SELECT, 0, 0)

    def call(n_layers=n, descs=descs, n_slots=2, stride=4000, dws_b=dws, sws_b=sws, side=FAKE + 16,
             lse=None, ks=2048, events=None, head_mask=None, frac=0.25, seg=(None, None, None)):
        return L.sfi_slow_step_layers(
            n_layers, descs, ptrs(n), ptrs(n), lse if lse is not None else ptrs(n), n_slots,
            ptrs(2), stride, ptrs(2), sws_b, FAKE, dws_b, 4, 256, ks, ptrs(n), 2052, ptrs(n),
            ctypes.c_float(frac), head_mask, *seg, FAKE, side,
            events if events is not None else ptrs(2), FAKE, FAKE)

    assert call(n_layers=0) == B.SFI_E_INVALID
    assert call(n_slots=0) == B.SFI_E_INVALID
    assert call(side=FAKE) == B.SFI_E_INVALID                 # the two streams must differ
    assert call(events=(ctypes.c_void_p * 2)(FAKE, None)) == B.SFI_E_INVALID
    assert call(lse=(ctypes.c_void_p * n)(FAKE, None, FAKE)) == B.SFI_E_INVALID
    assert call(dws_b=4096) == B.SFI_E_WORKSPACE
    assert call(sws_b=4096) == B.SFI_E_WORKSPACE
    assert call(stride=4002) == B.SFI_E_INVALID               # logits stride not a multiple of 4
    assert call(ks=5000) == B.SFI_E_INVALID                   # idx_stride < n_sink + k_sel
    assert call(head_mask=ptrs(n), frac=1.5) == B.SFI_E_INVALID
    bad = (B.sfi_kv_desc * n)(_desc(), _desc(), _desc(head_dim=96))
    assert call(descs=bad) == B.SFI_E_UNSUPPORTED             # the last layer is checked too
    assert call(seg=(ptrs(n), None, ptrs(n))) == B.SFI_E_INVALID       # all three or none
    assert call(seg=(ptrs(n), ptrs(n), (ctypes.c_void_p * n)(FAKE, FAKE, None))) == B.SFI_E_INVALID
    assert call(seg=(ptrs(n), ptrs(n, FAKE + 8), ptrs(n))) == B.SFI_E_INVALID   # alignment


def test_group_dot_validation(L):
    ok = dict(rows=FAKE, n=1 << 12, q=FAKE, G=4, unit=1, wg=64, part=FAKE, sink=FAKE)

    def call(**kw):
        a = {**ok, **kw}
        return L.sfi_group_dot(a["rows"], a["n"], a["q"], a["G"], a["unit"], a["wg"], a["part"],
                               a["sink"], None)
    assert call(rows=None) == B.SFI_E_INVALID
    assert call(q=None) == B.SFI_E_INVALID
    assert call(sink=None) == B.SFI_E_INVALID
    assert call(n=0) == B.SFI_E_INVALID
    assert call(n=(1 << 12) + 8) == B.SFI_E_INVALID           # whole 16-row groups only
    assert call(rows=FAKE + 8) == B.SFI_E_INVALID              # 16-byte loads
    assert call(q=FAKE + 4) == B.SFI_E_INVALID
    assert call(unit=3) == B.SFI_E_INVALID
    assert call(unit=-1) == B.SFI_E_INVALID
    assert call(wg=0) == B.SFI_E_INVALID
    assert call(wg=(1 << 20) + 1) == B.SFI_E_INVALID
    assert call(part=None) == B.SFI_E_INVALID                  # units 1 and 2 write it
    assert call(unit=2, part=None) == B.SFI_E_INVALID
    for G in (0, 3, 5, 16):
        assert call(G=G) == B.SFI_E_UNSUPPORTED


def test_stream_read_validation(L):
    assert L.sfi_stream_read(None, 1 << 20, 1024, FAKE, None) == B.SFI_E_INVALID
    assert L.sfi_stream_read(FAKE, 1 << 20, 1024, None, None) == B.SFI_E_INVALID
    assert L.sfi_stream_read(FAKE, 0, 1024, FAKE, None) == B.SFI_E_INVALID
    assert L.sfi_stream_read(FAKE, (1 << 20) + 8, 1024, FAKE, None) == B.SFI_E_INVALID
    assert L.sfi_stream_read(FAKE + 8, 1 << 20, 1024, FAKE, None) == B.SFI_E_INVALID
    assert L.sfi_stream_read(FAKE, 1 << 20, 1024, FAKE + 2, None) == B.SFI_E_INVALID
    assert L.sfi_stream_read(FAKE, 1 << 20, 0, FAKE, None) == B.SFI_E_INVALID
    assert L.sfi_stream_read(FAKE, 1 << 20, (1 << 20) + 1, FAKE, None) == B.SFI_E_INVALID


def test_gather_read_validation(L):
    d = _desc()
    gr = lambda dd=d, idx=FAKE, istride=2052, nidx=FAKE, nr=256, wg=256, sink=FAKE: \
        L.sfi_gather_read(ctypes.byref(dd), idx, istride, nidx, nr, wg, sink, None)
    assert gr(idx=None) == B.SFI_E_INVALID
    assert gr(nidx=None) == B.SFI_E_INVALID
    assert gr(sink=None) == B.SFI_E_INVALID
    assert gr(istride=0) == B.SFI_E_INVALID
    assert gr(nr=-1) == B.SFI_E_INVALID
    assert gr(wg=0) == B.SFI_E_INVALID
    assert gr(dd=_desc(head_dim=96)) == B.SFI_E_UNSUPPORTED


def test_reorg_and_two_segment_validation(L):
    d = _desc()
    D = ctypes.byref(d)
    ro = lambda **k: L.sfi_reorg(D, k.get("idx", FAKE), k.get("istride", 2052), FAKE,
                                 k.get("ck", FAKE), k.get("cv", FAKE), k.get("cpos", FAKE), None)
    assert ro(idx=None) == B.SFI_E_INVALID
    assert ro(ck=None) == B.SFI_E_INVALID
    assert ro(cpos=None) == B.SFI_E_INVALID
    assert ro(cv=FAKE + 8) == B.SFI_E_INVALID
    assert ro(cpos=FAKE + 2) == B.SFI_E_INVALID
    assert ro(istride=0) == B.SFI_E_INVALID
    assert ro(istride=1 << 30) == B.SFI_E_UNSUPPORTED          # 2*8*2^30 segment rows
    assert L.sfi_reorg(None, FAKE, 2052, FAKE, FAKE, FAKE, FAKE, None) == B.SFI_E_INVALID
    ws = L.sfi_workspace_bytes(D, B.SFI_OP_SPARSE, 2052, 256)
    sc = lambda **k: L.sfi_sparse_decode_compact(
        D, FAKE, k.get("ck", FAKE), k.get("cv", FAKE), k.get("cpos", FAKE),
        k.get("istride", 2052), FAKE, 256, None, FAKE, None, FAKE, k.get("ws", ws), None)
    assert sc(ck=None) == B.SFI_E_INVALID
    assert sc(cv=None) == B.SFI_E_INVALID
    assert sc(ck=FAKE + 4) == B.SFI_E_INVALID
    assert sc(cpos=None) == B.SFI_E_INVALID
    assert sc(ws=ws - 256) == B.SFI_E_WORKSPACE


def test_select_refined_validation(L):
    d = _desc()
    D = ctypes.byref(d)
    ws = L.sfi_workspace_bytes(D, B.SFI_OP_SELECT_REFINED, 0, 0)
    assert ws > L.sfi_workspace_bytes(D, B.SFI_OP_SELECT, 0, 0)

    def call(ws_bytes=ws, norm=FAKE, nstride=4000, **kw):
        pr = dict(B.REFINE_DEFAULTS)
        pr.update(kw)
        p = B.sfi_refine(pr["lambda_"], pr["alpha_soft"], pr["alpha_cross"], pr["prior_decay"],
                         pr["tail_frac"], pr["tail_brake"])
        return L.sfi_select_refined(D, FAKE, 4000, norm, nstride, 4, 64, 100, ctypes.byref(p),
                                    FAKE, 104, FAKE, FAKE, ws_bytes, None)

    assert call(lambda_=1.0) == B.SFI_E_INVALID
    assert call(lambda_=-0.1) == B.SFI_E_INVALID
    assert call(alpha_soft=1.0) == B.SFI_E_INVALID
    assert call(alpha_cross=float("nan")) == B.SFI_E_INVALID
    assert call(tail_frac=1.5) == B.SFI_E_INVALID
    assert call(prior_decay=-1.0) == B.SFI_E_INVALID
    assert call(nstride=3999) == B.SFI_E_INVALID
    assert call(ws_bytes=ws - 256) == B.SFI_E_WORKSPACE
    assert L.sfi_select_refined(D, FAKE, 4000, None, 0, 4, 64, 100, None, FAKE, 104, FAKE, FAKE,
                                ws, None) == B.SFI_E_INVALID
