"""Host-side parts of the interference probe (CPU)."""
import gc

from shard_placement_amd import probe


def test_timed_regions_pause_the_garbage_collector():
    assert gc.isenabled()
    with probe._no_gc():
        assert not gc.isenabled()
    assert gc.isenabled()
    try:
        with probe._no_gc():
            raise KeyError("x")
    except KeyError:
        pass
    assert gc.isenabled()
    gc.disable()
    try:
        with probe._no_gc():
            assert not gc.isenabled()
        assert not gc.isenabled()  # left as the caller had it
    finally:
        gc.enable()


def test_standalone_probe_needs_a_gpu():
    import pytest
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with pytest.raises(SystemExit, match="needs a GPU"):
        probe.main(["--workload", "1"])
