"""The clock probe (a measurement helper of the library) on the GPU: its
two counters give a plausible graphics clock, alone and beside running
attention kernels."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_clock_probe_reads_a_plausible_clock():
    import torch
    import causal_attention_amd as ca
    from tests.gpu_util import log, run_hip, to_device
    from workload import CONFIGS, make_inputs
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    ca.clock_probe(out, 2_000_000)  # 20 ms
    torch.cuda.synchronize()
    cycles, ticks = out.cpu().tolist()
    mhz = cycles / ticks * 100.0
    log(f"[clock] idle probe: {mhz:.0f} MHz over {ticks / 1e5:.1f} ms")
    assert ticks >= 2_000_000 and 300.0 < mhz < 3000.0
    # beside attention kernels on another stream
    x = make_inputs(CONFIGS["lm237m_ctx1024"], 3)
    dev = to_device(x)
    side = torch.cuda.Stream()
    ca.clock_probe(out, 500_000, stream=side)
    for _ in range(10):
        run_hip(x, dev=dev)
    torch.cuda.synchronize()
    cycles, ticks = out.cpu().tolist()
    mhz = cycles / ticks * 100.0
    log(f"[clock] under load: {mhz:.0f} MHz")
    assert 300.0 < mhz < 3000.0
