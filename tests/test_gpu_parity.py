"""HIP path vs the fp64 oracle on the one-layer workloads (full size) - needs the GPU."""
import pytest

from workloads import configs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl", [configs.TINY_2K_F32, configs.CTX8K_MHA, configs.CTX16K_GQA],
                         ids=lambda w: w.name)
def test_one_layer_step(wl):
    import gpu_cases
    gpu_cases.log(f"case {wl.name}")
    res = gpu_cases.one_layer_step(wl)
    gpu_cases.log(f"{wl.name}: " + ", ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}"
                                             for k, v in res.items()))
