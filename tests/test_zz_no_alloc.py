"""The allocation-free block scoring entry point against the workspace one, through the C ABI.

fdl_block_score_topc_noalloc keeps its workspace in a device array inside the library; its
block lists, relevance and block means must equal fdl_block_score_topc's bit for bit, on two
calls in a row (the second smaller, so it runs over the first call's leftover contents),
with the means computed from the keys and from means given.
"""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


def F():
    import long_context_diffusion_amd as lib
    return lib


def _case(seed, B, Hq, Hkv, L, P, d, bs, C, nq_max, dtype=torch.bfloat16):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    q = (torch.randn((B, Hq, L, d), generator=g, device=DEV) * 0.5).to(dtype)
    k = (torch.randn((B, Hkv, L, d), generator=g, device=DEV) * 0.5).to(dtype)
    gen = torch.Generator().manual_seed(seed)
    rows = torch.stack([torch.randperm(L, generator=gen)[:nq_max].sort().values for _ in range(B)]).to(torch.int32)
    n_q = torch.tensor([nq_max - (b % 3) for b in range(B)], dtype=torch.int32)
    return q, k, rows.to(DEV), n_q.to(DEV)


def _call_both(q, k, rows, n_q, P, bs, C, with_keys):
    lib = F().fdl.lib()
    fd = F().fdl
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    nq_max = rows.shape[1]
    nb = -(-P // bs)
    dt = fd.FDL_BF16 if q.dtype == torch.bfloat16 else fd.FDL_F32
    outs = []
    kbar_given = None if with_keys else F().block_means(k, P, bs)
    for noalloc in (False, True):
        blocks = torch.full((B, C), -7, dtype=torch.int32, device=DEV)
        R = torch.zeros((B, nb), dtype=torch.float64, device=DEV)
        kbar = torch.zeros((B, Hkv, nb, d), dtype=torch.float32, device=DEV) if with_keys else kbar_given.clone()
        kp = fd._ptr(k) if with_keys else None
        ks = fd._strides4(k) if with_keys else fd.Strides(0, 0, d)
        args = (dt, B, Hq, Hkv, L, P, d, fd._ptr(q), fd._strides4(q), fd._ptr(rows), fd._ptr(n_q), nq_max,
                kp, ks, ctypes.c_float(0.0), bs, C, fd._ptr(blocks), fd._ptr(R), fd._ptr(kbar))
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if noalloc:
            st = lib.fdl_block_score_topc_noalloc(*args, stream)
        else:
            need = lib.fdl_block_score_topc_workspace_bytes(dt, B, Hq, Hkv, P, d, bs, nq_max)
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
            st = lib.fdl_block_score_topc(*args, ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(need), stream)
        assert st == 0, fd.STATUS.get(st, st)
        torch.cuda.synchronize()
        outs.append((blocks, R, kbar))
    (b0, r0, k0), (b1, r1, k1) = outs
    assert torch.equal(b0, b1), "block lists differ"
    assert torch.equal(r0, r1), "relevance differs"
    assert torch.equal(k0, k1), "block means differ"
    return b1


@pytest.mark.parametrize("with_keys", [True, False])
def test_noalloc_matches_workspace_entry_point(with_keys):
    # first call: a larger input (32 KV heads, 252 blocks of 128 keys: the 32K step's shape,
    # 4.2 MB of workspace); second call: smaller, over the first one's leftovers
    q, k, rows, n_q = _case(1, 1, 32, 32, 32768, 32256, 128, 128, 64, 64)
    b = _call_both(q, k, rows, n_q, 32256, 128, 64, with_keys)
    assert int((b[0] >= 0).sum()) == 64
    q, k, rows, n_q = _case(2, 3, 8, 2, 3000, 2900, 64, 48, 11, 40)
    _call_both(q, k, rows, n_q, 2900, 48, 11, with_keys)


def test_noalloc_rejects_oversized_workspace():
    lib = F().fdl.lib()
    fd = F().fdl
    cap = lib.fdl_block_score_topc_noalloc_max_bytes()
    assert cap == 8 << 20
    # 8 sequences x 64 KV heads x 2000 blocks of d = 128 means: far above the cap
    need = lib.fdl_block_score_topc_workspace_bytes(fd.FDL_BF16, 8, 64, 64, 128000, 128, 64, 16)
    assert need > cap
    q = torch.zeros((1, 1, 1, 128), dtype=torch.bfloat16, device=DEV)
    st = lib.fdl_block_score_topc_noalloc(fd.FDL_BF16, 8, 64, 64, 128064, 128000, 128, fd._ptr(q),
                                          fd.Strides(0, 0, 128), None, None, 16, fd._ptr(q), fd.Strides(0, 0, 128),
                                          ctypes.c_float(0.0), 64, 4, fd._ptr(q), None, None,
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 5   # FDL_ERR_WORKSPACE, before any launch
