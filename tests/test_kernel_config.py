"""Pins of the host-side kernel-configuration mirror (tests/kernel_config.py)
to the thresholds the library header states for row invariance across M."""
from kernel_config import mfma_configuration, register_persistent_fits


def groups(N, K, bits, gs, cus=256):
    out = {}
    for M in range(1, 17):
        out.setdefault(mfma_configuration(M, N, K, bits, gs, cus), []).append(M)
    return sorted(out.values())


def test_down_projection_has_three_configurations():
    # K = 17408, N = 5120, 4-bit, group size 128 (the header's example)
    assert groups(5120, 17408, 4, 128) == [list(range(1, 8)), list(range(8, 15)), [15, 16]]


def test_register_persistent_reach():
    assert register_persistent_fits(4096, 4, 64) and not register_persistent_fits(4352, 4, 64)
    assert register_persistent_fits(6144, 4, 128) and not register_persistent_fits(6656, 4, 128)
    assert register_persistent_fits(6144, 2, 64) and not register_persistent_fits(6400, 2, 64)


def test_shapes_within_reach_have_one_configuration():
    # gate/up of the same layer and a square shape: one configuration for all M
    assert len(groups(17408, 5120, 4, 128)) == 1
    assert len(groups(4096, 4096, 4, 64)) == 1
