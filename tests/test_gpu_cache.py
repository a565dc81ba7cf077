"""Approximate-KV refresh and block-means refresh on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import focus_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"


def F():
    import long_context_diffusion_amd as lib
    return lib


def f64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def _rand(g, shape, dtype):
    return torch.randn(shape, generator=g, device=DEV).to(dtype)


@pytest.mark.parametrize("dtype,d,with_vt", [(torch.float32, 64, False), (torch.bfloat16, 64, False),
                                             (torch.bfloat16, 128, True)])
def test_kv_and_means_refresh_small(dtype, d, with_vt):
    B, Hkv, L, P, bs = 2, 2, 304, 250, 16
    g = torch.Generator(device=DEV)
    g.manual_seed(d)
    k, v = _rand(g, (B, Hkv, L, d), dtype), _rand(g, (B, Hkv, L, d), dtype)
    rows = torch.tensor([[3, 4, 40, 47, 48, 199, 245, 249, 250, 290, 7, 8],
                         [0, 15, 16, -1, 100, 303, 9, 9, 9, 9, 9, 9]], dtype=torch.int32, device=DEV)
    n_rows = torch.tensor([10, 6], dtype=torch.int32, device=DEV)   # entries past n_rows are ignored
    n_max = rows.shape[1]
    k_new, v_new = _rand(g, (B, Hkv, n_max, d), dtype), _rand(g, (B, Hkv, n_max, d), dtype)
    kf, vf = f64(k), f64(v)
    kbar = F().block_means(k, P, bs)
    kbar_old = kbar.clone()
    vt = F().transpose_v(v) if with_vt else None
    F().kv_refresh(rows, k_new, v_new, k, v, n_rows=n_rows, vt=vt)
    F().block_means_refresh(k, P, bs, rows, kbar, n_rows=n_rows)
    torch.cuda.synchronize()
    for b in range(B):
        n = int(n_rows[b])
        r = rows[b, :n].cpu().numpy()
        K2, V2 = O.kv_refresh(kf[b], vf[b], r, f64(k_new)[b][:, :n], f64(v_new)[b][:, :n])
        assert np.array_equal(f64(k)[b], K2) and np.array_equal(f64(v)[b], V2), f"cache b{b}"
        ref = O.block_means(K2, P, bs).astype(np.float32)
        assert np.array_equal(kbar[b].cpu().numpy(), ref), f"means b{b}"
        untouched = np.setdiff1d(np.arange(ref.shape[1]), O.refreshed_blocks(r, P, bs))
        assert torch.equal(kbar[b][:, untouched], kbar_old[b][:, untouched])
    if with_vt:
        assert torch.equal(vt, v.transpose(2, 3))


def test_refresh_at_32k_with_active_rows():
    """U(t) = I_active of the 32K step; then scoring and sparse attention read the refreshed
    cache: the means equal the oracle's on every touched block and stay as they were elsewhere."""
    import gpu_cases
    from workloads import configs, synth
    wl = configs.CTX32K_STACK
    conf, mask = synth.step_inputs(wl)
    _, _, active, n_active = gpu_cases.gpu_select(wl, conf, mask, DEV)
    k, v = synth.make_kv(wl, 2, DEV)
    vt = F().transpose_v(v)
    kbar = F().block_means(k, wl.P, wl.bs)
    kbar_old = kbar.clone()
    g = torch.Generator(device=DEV)
    g.manual_seed(32)
    n_max = active.shape[1]
    k_new = _rand(g, (wl.B, wl.Hkv, n_max, wl.d), k.dtype)
    v_new = _rand(g, (wl.B, wl.Hkv, n_max, wl.d), v.dtype)
    F().kv_refresh(active, k_new, v_new, k, v, n_rows=n_active, vt=vt)
    F().block_means_refresh(k, wl.P, wl.bs, active, kbar, n_rows=n_active)
    torch.cuda.synchronize()
    na = int(n_active[0])
    r = active[0, :na].cpu().numpy()
    kn, vn = f64(k_new[0]), f64(v_new[0])
    for j in np.linspace(0, na - 1, 16).astype(int):
        assert np.array_equal(f64(k[0][:, int(r[j])]), kn[:, j]) and np.array_equal(f64(v[0][:, int(r[j])]), vn[:, j])
        assert torch.equal(vt[0][:, :, int(r[j])], v[0][:, int(r[j])])
    touched = O.refreshed_blocks(r, wl.P, wl.bs)
    kf = f64(k[0])
    for blk in touched:
        lo, hi = blk * wl.bs, min((blk + 1) * wl.bs, wl.P)
        ref = O.block_means(kf[:, lo:hi], hi - lo, hi - lo)[:, 0].astype(np.float32)
        assert np.array_equal(kbar[0][:, blk].cpu().numpy(), ref), f"block {blk}"
    untouched = np.setdiff1d(np.arange(wl.nb), touched)
    assert torch.equal(kbar[0][:, untouched], kbar_old[0][:, untouched])
    gpu_cases.log(f"refresh: {na} rows, {len(touched)} prompt blocks touched")
