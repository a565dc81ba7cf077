"""The C ABI on the host: exports, status strings, workspace sizes and argument validation.

Nothing here launches a kernel: every call below is rejected by host-side
validation before any HIP call, or is a pure host query.  Pointers passed are
fake, aligned (or deliberately misaligned) integers that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from long_context_diffusion_amd import fdl as F
from oracle import focus_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fdl.h")

FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10008)
NULL = None
S = F.Strides


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fdl_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = F.lib()
    names = declared_functions()
    assert len(names) == len(F.EXPORTS), names
    assert sorted(F.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in range(8):
        s = F.lib().fdl_status_string(code)
        assert s and len(s) > 1
    assert F.lib().fdl_status_string(0) == b"ok"


@pytest.mark.parametrize("n_t,rho", [(4, 2.0), (3, 2.5), (16, 4.0), (0, 4.0), (5, 0.1), (10, 0.3),
                                      (7, 1.0 / 3.0), (1000, 0.999)])
def test_focus_count_matches_oracle(n_t, rho):
    assert F.focus_count(n_t, rho) == O.focus_count(n_t, rho)


def test_focus_count_rejects_negative():
    assert F.focus_count(-1, 2.0) == 0
    assert F.focus_count(3, -1.0) == 0


def test_workspace_sizes():
    lib = F.lib()
    # bf16 d = 128: the split count is picked on the device from the valid rows, so the
    # workspace covers fp32 partials of at most 512 work items of 256 rows, whatever
    # nq_max is
    cap = 512 * 256 * (128 + 2) * 4
    for nq_max in (1024, 32768):
        n = lib.fdl_dense_attention_workspace_bytes(F.FDL_BF16, 1, 32, 32, 32768, 128, nq_max)
        assert n == cap
    # a short key range leaves nothing to split
    assert lib.fdl_dense_attention_workspace_bytes(F.FDL_BF16, 1, 32, 32, 512, 128, 1024) == 0
    # fp32 splits per row: at least two splits of fp32 partials for <= 1024 active rows
    n = lib.fdl_dense_attention_workspace_bytes(F.FDL_F32, 1, 32, 32, 32768, 128, 1024)
    assert n >= 2 * 32 * 1024 * (128 + 2) * 4
    assert lib.fdl_sparse_attention_workspace_bytes(F.FDL_BF16, 1, 32, 32, 32768, 32256, 128,
                                                     1024, 16, 64, 128) > 0
    # sinks: the partial scores, then room for the lse pass it runs when given no lse (lse and
    # output rows of the active queries, and that dense pass's own workspace)
    def r256_(x):
        return -(-x // 256) * 256
    assert lib.fdl_sink_identify_workspace_bytes(F.FDL_BF16, 1, 32, 32, 32768, 128, 1024) == \
        r256_((32 * 32768 + 32768) * 4) + r256_(32 * 1024 * 4) + r256_(32 * 1024 * 128 * 2) + cap
    # block scoring: each KV head's part of R, R, and room for the block means when they are
    # computed from the keys; the number of query rows does not change it
    nb = 252

    def r256(x):
        return -(-x // 256) * 256
    for nq_max in (1024, 100, 1 << 20):
        assert lib.fdl_block_score_topc_workspace_bytes(F.FDL_BF16, 1, 32, 32, 32256, 128, 128, nq_max) == \
            r256(32 * nb * 8) + r256(nb * 8) + 32 * nb * 128 * 4
    # invalid shapes report 0
    assert lib.fdl_dense_attention_workspace_bytes(F.FDL_BF16, 1, 32, 5, 1024, 128, 64) == 0
    assert lib.fdl_block_score_topc_workspace_bytes(F.FDL_BF16, 1, 4, 4, 0, 64, 64, 16) == 0


def _pcgi(**kw):
    args = dict(conf=FAKE, mask=FAKE, B=1, L=2048, n_t=4, rho=2.0, w=8, focus=FAKE, n_focus=FAKE,
                k_cap=8, active=FAKE, n_active=FAKE, nq_max=64)
    args.update(kw)
    return F.lib().fdl_pcgi_select(args["conf"], args["mask"], args["B"], args["L"], args["n_t"],
                                   args["rho"], args["w"], args["focus"], args["n_focus"], args["k_cap"],
                                   args["active"], args["n_active"], args["nq_max"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(conf=NULL), 1), (dict(active=NULL), 1), (dict(n_focus=NULL), 1),
    (dict(B=0), 2), (dict(L=0), 2), (dict(w=0), 2), (dict(n_t=-1), 2), (dict(rho=float("nan")), 2),
    (dict(rho=-1.0), 2), (dict(rho=float("inf")), 2),
    (dict(k_cap=7), 2),            # k = 8 needs k_cap >= 8
    (dict(nq_max=63), 2),          # k*w = 64 active positions at most
])
def test_pcgi_validation(kw, status):
    assert _pcgi(**kw) == status


def _dense(**kw):
    a = dict(dt=F.FDL_BF16, B=1, Hq=4, Hkv=4, L=256, d=128, q=FAKE, qs=S(4 * 256 * 128, 256 * 128, 128),
             q_idx=NULL, n_q=NULL, nq_max=256, k=FAKE, ks=S(4 * 256 * 128, 256 * 128, 128), v=FAKE,
             vs=S(4 * 256 * 128, 256 * 128, 128), vt=NULL, vts=S(0, 0, 0), scale=0.0, o=FAKE,
             os=S(4 * 256 * 128, 256 * 128, 128), lse=NULL, ws=NULL, ws_bytes=0)
    a.update(kw)
    return F.lib().fdl_dense_attention(a["dt"], a["B"], a["Hq"], a["Hkv"], a["L"], a["d"], a["q"], a["qs"],
                                       a["q_idx"], a["n_q"], a["nq_max"], a["k"], a["ks"], a["v"], a["vs"],
                                       a["vt"], a["vts"], a["scale"], a["o"], a["os"], a["lse"], a["ws"],
                                       a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), 1), (dict(k=NULL), 1), (dict(v=NULL), 1), (dict(o=NULL), 1),
    (dict(dt=2), 3), (dict(dt=-1), 3),
    (dict(d=96), 7), (dict(d=256), 7),
    (dict(Hkv=3), 2), (dict(B=0), 2), (dict(L=0), 2), (dict(nq_max=-1), 2),
    (dict(q=MISALIGNED), 4), (dict(ks=S(4 * 256 * 128, 256 * 128, 132)), 4),
    (dict(qs=S(4 * 256 * 128, 256 * 128, 64)), 2),       # rows overlap: |row stride| < d
    (dict(vs=S(0, 0, 1 << 31)), 2), (dict(ks=S(0, 0, -(1 << 31))), 2),   # row stride beyond 2^31
    (dict(nq_max=16, L=4096), 5),                        # few rows -> key split needs a workspace
    (dict(nq_max=16, L=4096, ws=FAKE, ws_bytes=64), 5),
    (dict(nq_max=16, L=4096, ws=MISALIGNED, ws_bytes=1 << 30), 4),
    (dict(nq_max=0), 0),                                 # nothing to compute
    # V^T: checked for the bf16 d = 128 path only, before anything runs
    (dict(nq_max=0, vt=MISALIGNED, vts=S(0, 0, 256)), 4),
    (dict(nq_max=0, vt=FAKE, vts=S(0, 0, 260)), 4),      # d-row stride not a multiple of 8
    (dict(nq_max=0, vt=FAKE, vts=S(4, 0, 256)), 4),
    (dict(nq_max=0, vt=FAKE, vts=S(0, 0, 248)), 2),      # d rows shorter than L
    (dict(nq_max=0, vt=FAKE, vts=S(0, 0, 1 << 24)), 2),
    (dict(nq_max=0, vt=FAKE, vts=S(128 * 256, 256, 256)), 0),
    (dict(nq_max=0, dt=F.FDL_F32, vt=MISALIGNED, vts=S(0, 0, 3)), 0),   # fp32: V^T is not read or checked
])
def test_dense_validation(kw, status):
    if status == 5 or status == 4 and "ws" in kw:
        # these rows must reach the workspace check, i.e. the plan really splits the keys
        assert F.lib().fdl_dense_attention_workspace_bytes(F.FDL_BF16, 1, 4, 4, kw["L"], 128, 16) > 0
    assert _dense(**kw) == status


def test_sparse_and_sink_and_block_validation():
    lib = F.lib()
    st = S(4 * 256 * 128, 256 * 128, 128)
    # sparse: the key list always needs a workspace
    assert lib.fdl_sparse_attention(F.FDL_BF16, 1, 4, 4, 256, 192, 128, FAKE, st, NULL, NULL, 64, FAKE, st,
                                    FAKE, st, NULL, S(0, 0, 0), FAKE, 4000, FAKE, 2, 64, 0.0, FAKE, st, NULL, NULL, 0,
                                    None) == 5
    # sparse: sink or block lists longer than the device canonicalises (4096 entries)
    for n_sinks, C in ((4097, 2), (4, 4097)):
        assert lib.fdl_sparse_attention(F.FDL_BF16, 1, 4, 4, 256, 192, 128, FAKE, st, NULL, NULL, 64, FAKE, st,
                                        FAKE, st, NULL, S(0, 0, 0), FAKE, n_sinks, FAKE, C, 64, 0.0, FAKE, st, NULL,
                                        NULL, 0, None) == 7
    # sparse: P > L, bs < 1, block list missing
    assert lib.fdl_sparse_attention(F.FDL_BF16, 1, 4, 4, 256, 300, 128, FAKE, st, NULL, NULL, 64, FAKE, st,
                                    FAKE, st, NULL, S(0, 0, 0), FAKE, 4, FAKE, 2, 64, 0.0, FAKE, st, NULL, NULL, 0, None) == 2
    assert lib.fdl_sparse_attention(F.FDL_BF16, 1, 4, 4, 256, 192, 128, FAKE, st, NULL, NULL, 64, FAKE, st,
                                    FAKE, st, NULL, S(0, 0, 0), FAKE, 4, FAKE, 2, 0, 0.0, FAKE, st, NULL, NULL, 0, None) == 2
    assert lib.fdl_sparse_attention(F.FDL_BF16, 1, 4, 4, 256, 192, 128, FAKE, st, NULL, NULL, 64, FAKE, st,
                                    FAKE, st, NULL, S(0, 0, 0), FAKE, 4, NULL, 2, 64, 0.0, FAKE, st, NULL, NULL, 0, None) == 1
    # sinks: lse and output required, n_sinks within [0, L], workspace
    # no lse: the library computes it, in a larger workspace than the one the scores alone need
    small = (4 * 256 + 256) * 4
    assert lib.fdl_sink_identify_workspace_bytes(F.FDL_BF16, 1, 4, 4, 256, 128, 64) > small
    assert lib.fdl_sink_identify(F.FDL_BF16, 1, 4, 4, 256, 128, FAKE, st, NULL, NULL, 64, FAKE, st, 0.0,
                                 NULL, 4, FAKE, NULL, FAKE, small, None) == 5
    assert lib.fdl_sink_identify(F.FDL_BF16, 1, 4, 4, 256, 128, FAKE, st, NULL, NULL, 64, FAKE, st, 0.0,
                                 FAKE, 4, NULL, NULL, FAKE, 1 << 20, None) == 1
    assert lib.fdl_sink_identify(F.FDL_BF16, 1, 4, 4, 256, 128, FAKE, st, NULL, NULL, 64, FAKE, st, 0.0,
                                 FAKE, 257, FAKE, NULL, FAKE, 1 << 20, None) == 2
    assert lib.fdl_sink_identify(F.FDL_BF16, 1, 4, 4, 256, 128, FAKE, st, NULL, NULL, 64, FAKE, st, 0.0,
                                 FAKE, 4, FAKE, NULL, FAKE, 16, None) == 5
    # blocks: P outside [1, L], C < 0, workspace too small
    for P, bs, C, ws_bytes, status in [(0, 64, 4, 1 << 20, 2), (257, 64, 4, 1 << 20, 2),
                                       (192, 0, 4, 1 << 20, 2), (192, 64, -1, 1 << 20, 2),
                                       (192, 64, 4, 8, 5)]:
        assert lib.fdl_block_score_topc(F.FDL_BF16, 1, 4, 4, 256, P, 128, FAKE, st, NULL, NULL, 64, FAKE, st,
                                        0.0, bs, C, FAKE, NULL, NULL, FAKE, ws_bytes, None) == status
    # blocks without keys need the precomputed means
    assert lib.fdl_block_score_topc(F.FDL_BF16, 1, 4, 4, 256, 192, 128, FAKE, st, NULL, NULL, 64, NULL, st,
                                    0.0, 64, 4, FAKE, NULL, NULL, FAKE, 1 << 20, None) == 1
    # block means: output required, P within [1, L], bs >= 1, aligned keys
    for kw_, status in [(dict(kbar=NULL), 1), (dict(P=0), 2), (dict(P=257), 2), (dict(bs=0), 2),
                        (dict(k=MISALIGNED), 4), (dict(k=NULL), 1), (dict(Hkv=0), 2)]:
        a = dict(B=1, Hkv=4, L=256, P=192, d=128, k=FAKE, bs=64, kbar=FAKE)
        a.update(kw_)
        assert lib.fdl_block_means(F.FDL_BF16, a["B"], a["Hkv"], a["L"], a["P"], a["d"], a["k"], st, a["bs"],
                                   a["kbar"], None) == status, kw_


def test_vt_marshalling():
    """The binding passes V^T as (pointer, (b, h, d) strides) and rejects a tensor that is
    not V's [B, Hkv, d, L] transpose; transpose_v pads rows to 8 keys (aligned strides)."""
    import torch
    from long_context_diffusion_amd import fdl
    v = torch.zeros((2, 3, 13, 128), dtype=torch.bfloat16)
    vt = fdl.transpose_v(v)
    assert tuple(vt.shape) == (2, 3, 128, 13) and vt.stride(3) == 1
    assert vt.stride(2) == 16 and vt.stride(1) == 128 * 16 and vt.stride(0) == 3 * 128 * 16
    assert torch.equal(vt, v.transpose(2, 3))
    ptr, st = fdl._vt(vt, v)
    assert ptr.value == vt.data_ptr() and (st.b, st.h, st.r) == (3 * 128 * 16, 128 * 16, 16)
    assert fdl._vt(None, v)[0] is None
    with pytest.raises(fdl.FdlError):
        fdl._vt(v, v)                                   # not transposed
    with pytest.raises(fdl.FdlError):
        fdl._vt(vt.to(torch.float32), v)                # dtype differs


def test_kv_refresh_validation():
    lib = F.lib()
    st = S(4 * 256 * 128, 256 * 128, 128)
    z = S(0, 0, 0)
    # rows missing, sizes, dtype, alignment; nothing to do with n_max = 0
    assert lib.fdl_kv_refresh(F.FDL_BF16, 1, 4, 256, 128, NULL, NULL, 8, FAKE, st, FAKE, st, FAKE, st, FAKE, st,
                              NULL, z, None) == 1
    assert lib.fdl_kv_refresh(F.FDL_BF16, 1, 4, 256, 128, FAKE, NULL, -1, FAKE, st, FAKE, st, FAKE, st, FAKE, st,
                              NULL, z, None) == 2
    assert lib.fdl_kv_refresh(F.FDL_BF16, 1, 4, 256, 96, FAKE, NULL, 8, FAKE, st, FAKE, st, FAKE, st, FAKE, st,
                              NULL, z, None) == 7
    assert lib.fdl_kv_refresh(F.FDL_BF16, 1, 4, 256, 128, FAKE, NULL, 8, FAKE, st, FAKE, st, MISALIGNED, st, FAKE,
                              st, NULL, z, None) == 4
    assert lib.fdl_kv_refresh(F.FDL_BF16, 1, 4, 256, 128, FAKE, NULL, 0, FAKE, st, FAKE, st, FAKE, st, FAKE, st,
                              FAKE, S(0, 0, 248), None) == 2          # V^T rows shorter than L
    assert lib.fdl_kv_refresh(F.FDL_BF16, 1, 4, 256, 128, FAKE, NULL, 0, FAKE, st, FAKE, st, FAKE, st, FAKE, st,
                              NULL, z, None) == 0
    # block means refresh: kbar and rows required, P within [1, L], bs >= 1
    assert lib.fdl_block_means_refresh(F.FDL_BF16, 1, 4, 256, 192, 128, FAKE, st, 64, FAKE, NULL, 8, NULL,
                                       None) == 1
    assert lib.fdl_block_means_refresh(F.FDL_BF16, 1, 4, 256, 192, 128, FAKE, st, 64, NULL, NULL, 8, FAKE,
                                       None) == 1
    assert lib.fdl_block_means_refresh(F.FDL_BF16, 1, 4, 256, 300, 128, FAKE, st, 64, FAKE, NULL, 8, FAKE,
                                       None) == 2
    assert lib.fdl_block_means_refresh(F.FDL_BF16, 1, 4, 256, 192, 128, FAKE, st, 0, FAKE, NULL, 8, FAKE,
                                       None) == 2
    assert lib.fdl_block_means_refresh(F.FDL_BF16, 1, 4, 256, 192, 128, FAKE, st, 64, NULL, NULL, 0, FAKE,
                                       None) == 0


def test_confidence_validation():
    lib = F.lib()
    ls = S(4 * 1024, 0, 1024)
    ws_n = lib.fdl_confidence_unmask_workspace_bytes(1, 1000, 4)
    assert ws_n == 4 * 1 * 16                                  # one (m, s, arg) part per row and chunk
    assert lib.fdl_confidence_unmask_workspace_bytes(1, 1000, 4097) == 0

    def call(dt=F.FDL_BF16, B=1, L=64, V=1000, logits=FAKE, s=ls, pos=FAKE, m_max=4, n_t=2, mask=FAKE,
             conf=FAKE, ws=FAKE, n=ws_n):
        return lib.fdl_confidence_unmask(dt, B, L, V, logits, s, pos, NULL, m_max, n_t, mask, conf, NULL, NULL,
                                         ws, n, None)
    assert call(dt=5) == 3
    assert call(n_t=-1) == 2 and call(V=0) == 2 and call(s=S(0, 0, 992)) == 2   # rows shorter than V
    assert call(m_max=4097) == 7
    assert call(mask=NULL) == 1 and call(pos=NULL) == 1
    assert call(logits=MISALIGNED) == 4 and call(s=S(0, 0, 1001)) == 4
    assert call(ws=NULL) == 5 and call(n=ws_n - 1) == 5
    assert call(m_max=0) == 0                                  # nothing listed: nothing to do


def test_dcu_validation():
    lib = F.lib()
    # the fp64 partial sums of 32-token groups of every (sequence, layer)
    assert lib.fdl_dcu_select_workspace_bytes(1, 32, 32768) == 32 * 1024 * 8
    assert lib.fdl_dcu_select_workspace_bytes(2, 3, 33) == 2 * 3 * 2 * 8
    assert lib.fdl_dcu_select_workspace_bytes(0, 3, 33) == 0
    xs = S(32 * 1024 * 4096, 1024 * 4096, 4096)
    ws_n = lib.fdl_dcu_select_workspace_bytes(1, 32, 1024)

    def call(dt=F.FDL_BF16, B=1, NL=32, L=1024, H=4096, xn=FAKE, sn=xs, xp=FAKE, sp=xs, keys=FAKE, n_keys=4,
             w_m=8, total=100, out=FAKE, ws=FAKE, n=ws_n):
        return lib.fdl_dcu_select(dt, B, NL, L, H, xn, sn, xp, sp, keys, n_keys, w_m, total, out, out, out, out,
                                  out, ws, n, None)
    assert call(dt=2) == 3
    assert call(H=0) == 2 and call(total=-1) == 2 and call(w_m=0) == 2 and call(n_keys=-1) == 2
    assert call(L=(1 << 18) + 1) == 7 and call(NL=1025) == 7
    assert call(xp=NULL) == 1 and call(out=NULL) == 1 and call(keys=NULL) == 1
    assert call(xn=MISALIGNED) == 4 and call(sp=S(0, 0, 4100)) == 4
    assert call(ws=NULL) == 5 and call(n=ws_n - 8) == 5


def test_variant_entry_points_validation():
    lib = F.lib()
    st = S(32 * 32768 * 128, 32768 * 128, 128)
    # a mode outside FDL_SCORE_PER_HEAD | FDL_SCORE_MAX, and blocks_per_head outside {0, 1}
    ws = lib.fdl_block_score_topc_workspace_bytes(F.FDL_BF16, 1, 32, 32, 32256, 128, 128, 1024)
    for mode, status in ((4, 2), (-1, 2)):
        assert lib.fdl_block_score_topc_ex(F.FDL_BF16, 1, 32, 32, 32768, 32256, 128, FAKE, st, FAKE, FAKE, 1024,
                                           FAKE, st, 0.0, 128, 64, mode, FAKE, NULL, NULL, FAKE, ws, None) == status
    assert lib.fdl_sparse_attention_ex_workspace_bytes(F.FDL_BF16, 1, 32, 32, 32768, 32256, 128, 1024, 16, 64,
                                                       128, 2) == 0
    z = S(0, 0, 0)
    assert lib.fdl_sparse_attention_ex(F.FDL_BF16, 1, 32, 32, 32768, 32256, 128, FAKE, st, FAKE, FAKE, 1024,
                                       FAKE, st, FAKE, st, NULL, z, FAKE, 16, FAKE, 64, 2, 128, 0.0, FAKE, st,
                                       NULL, FAKE, 1 << 30, None) == 2
    # per-head key lists: one list per (sequence, KV head) where the list path is taken
    shared = lib.fdl_sparse_attention_ex_workspace_bytes(F.FDL_F32, 2, 8, 4, 4096, 4000, 64, 256, 8, 16, 64, 0)
    ph = lib.fdl_sparse_attention_ex_workspace_bytes(F.FDL_F32, 2, 8, 4, 4096, 4000, 64, 256, 8, 16, 64, 1)
    assert ph > shared
    assert lib.fdl_sparse_attention_ex_workspace_bytes(F.FDL_F32, 2, 8, 4, 4096, 4000, 64, 256, 8, 16, 64, 0) == \
        lib.fdl_sparse_attention_workspace_bytes(F.FDL_F32, 2, 8, 4, 4096, 4000, 64, 256, 8, 16, 64)


def test_block_means_alignment():
    lib = F.lib()
    st = S(32 * 32768 * 128, 32768 * 128, 128)
    assert lib.fdl_block_means(F.FDL_BF16, 1, 32, 32768, 32256, 128, FAKE, st, 128, MISALIGNED, None) == 4
    assert lib.fdl_block_means_refresh(F.FDL_BF16, 1, 32, 32768, 32256, 128, FAKE, st, 128, FAKE, NULL, 8,
                                       MISALIGNED, None) == 4


def test_calibrate_validation():
    lib = F.lib()
    out = ctypes.c_void_p(0x20000)
    assert lib.fdl_calibrate_read(FAKE, 0, out, 8, NULL) == 2
    assert lib.fdl_calibrate_read(FAKE, 24, out, 8, NULL) == 2
    assert lib.fdl_calibrate_read(FAKE, 4096, out, 0, NULL) == 2
    assert lib.fdl_calibrate_read(NULL, 4096, out, 8, NULL) == 1
    assert lib.fdl_calibrate_read(FAKE, 4096, NULL, 8, NULL) == 1
    assert lib.fdl_calibrate_read(MISALIGNED, 4096, out, 8, NULL) == 4
    assert lib.fdl_calibrate_mfma(0, 10, 1.0, 1.0, out, NULL) == 2
    assert lib.fdl_calibrate_mfma(4, 0, 1.0, 1.0, out, NULL) == 2
    assert lib.fdl_calibrate_mfma(4, 10, 1.0, 1.0, NULL, NULL) == 1


def test_kv_refresh_means_validation():
    lib = F.lib()
    st = S(32 * 4096 * 128, 4096 * 128, 128)
    ns = S(32 * 64 * 128, 64 * 128, 128)
    kb = ctypes.c_void_p(0x40000)
    args = lambda P, bs, kbar: (F.FDL_BF16, 1, 32, 4096, P, 128, bs, FAKE, NULL, 64, FAKE, ns, FAKE, ns,
                                FAKE, st, FAKE, st, NULL, S(0, 0, 0), kbar, NULL)
    assert lib.fdl_kv_refresh_means(*args(4000, 4096, kb)) == 7     # block size above the fused bound
    assert lib.fdl_kv_refresh_means(*args(4097, 64, kb)) == 2
    assert lib.fdl_kv_refresh_means(*args(4000, 0, kb)) == 2
    assert lib.fdl_kv_refresh_means(*args(4000, 64, NULL)) == 1
    assert lib.fdl_kv_refresh_means(*args(4000, 64, MISALIGNED)) == 4
