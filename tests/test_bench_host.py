"""Host logic of bench.py that needs no GPU: the shader-clock sampler's parsing
of the amdgpu ``pp_dpm_sclk`` file and its behaviour without one."""

import importlib.util
import os
import time
import types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _props():
    return types.SimpleNamespace(pci_domain_id=0, pci_bus_id=0x75, pci_device_id=0)


def test_clock_sampler_reads_the_marked_level(tmp_path):
    bench = _bench()
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1911Mhz *\n2: 2400Mhz\n")
    cs = bench.ClockSampler(_props(), period=0.001)
    cs.path = str(f)            # point the sampler at the fixture
    assert cs._read() == 1911
    cs.start()
    time.sleep(0.02)
    assert cs.stop() == 1911.0


def test_clock_sampler_handles_no_marked_line_and_no_file(tmp_path):
    bench = _bench()
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 2400Mhz\n")
    cs = bench.ClockSampler(_props(), period=0.001)
    cs.path = str(f)
    assert cs._read() is None
    cs.start()
    time.sleep(0.01)
    assert cs.stop() is None    # no sample taken
    cs2 = bench.ClockSampler(_props())
    cs2.path = None             # no sysfs file on this machine
    assert cs2.start().stop() is None


def test_bench_tile_counts_match_oracle():
    """The map study's tile-level work (the kernel's 32-query x 64-key tile
    skip, from the library's maps) equals the oracle's tile_step_work."""
    import numpy as np
    import bench
    from oracle import partition as opart
    for kind in opart.KINDS:
        for N in (1, 2, 4, 8):
            S = 2 * N * 192
            got = np.array([bench.tile_pairs_per_step(kind, S, N, r) for r in range(N)])
            assert np.array_equal(got, opart.tile_step_work(kind, S, N, 32, 64)), (kind, N)
            got_el = np.array([bench.visible_pairs_per_step(kind, S, N, r, True) for r in range(N)])
            assert np.array_equal(got_el, opart.step_work(kind, S, N)), (kind, N)
