"""The unit-throughput probes behind bench.py's measured peaks return rates
between a conservative floor and the MI355X datasheet peak (256 CUs at
2.4 GHz): dense matrix cores 2516.6 TFLOP/s (bf16, fp16) and 157.3 TFLOP/s
(fp32), v_exp_f32 at 32 lanes per clock per CU, 19.66e12/s."""
import pytest

pytestmark = pytest.mark.gpu

# kind -> (datasheet peak, floor), per second
BOUNDS = {
    "mfma-bf16": (2516.6e12, 500e12),
    "mfma-fp16": (2516.6e12, 500e12),
    "mfma-fp32": (157.3e12, 30e12),
    "exp": (256 * 32 * 2.4e9, 4e12),
}


@pytest.mark.parametrize("kind", sorted(BOUNDS))
def test_probe_rate_is_plausible(fs, kind):
    import torch

    from streaming_sinkhorn_solver_amd import binding

    sink = torch.zeros(4, device="cuda")
    rate = binding.fs_probe_peak(kind, sink, reps=5)
    peak, floor = BOUNDS[kind]
    print(f"{kind}: {rate / 1e12:.1f} T/s ({rate / peak:.1%} of the datasheet peak)")
    assert floor <= rate <= 1.02 * peak
    assert float(sink[0]) == 0.0  # the probe's guarded store never fires
