"""Host-side helpers of bench.py that run without a GPU."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# amd-smi metric --clock --power, one GPU, cut to the fields the sampler reads
# (two of the eight shader-clock domains, the memory clock that must not count)
SMI_TEXT = """GPU: 0
    POWER:
        SOCKET_POWER: 1319 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1980 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 2000 MHz
            MIN_CLK: 500 MHz
        MEM_0:
            CLK: 2000 MHz
            MIN_CLK: 2000 MHz
        SOCCLK_0:
            CLK: 38 MHz
"""


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_power_sample_parse():
    b = _bench()
    assert b.PowerSampler.parse(SMI_TEXT) == (1319.0, 1990.0)
    assert b.PowerSampler.parse("GPU: 0\n    POWER:\n        SOCKET_POWER: N/A\n") is None


def test_power_sampler_off_returns_none():
    b = _bench()
    pw = b.PowerSampler(False)
    pw.start()
    assert pw.stop() is None
