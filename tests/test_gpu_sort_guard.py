"""The bounded look-back waits of the sort and of the intersection-count scans: with a spin limit of zero a
partition that does not find its predecessors' counts at the first look gives up, flags the device error word and
finishes, so every kernel still exits normally; gs_device_check then reports GS_ERR_DEVICE. With the default limit
the same work is exact and reports nothing. (The limit is set from the host; no workspace is corrupted to provoke
the failure.)

Semantics being guarded: gsplat 1.0.0 native extension, intersections.c, gs_isect_tiles turns a failure of its
sort into an error status (NoMemError) rather than returning a wrong order silently."""
import numpy as np
import pytest
import torch

from tile_binned_gaussian_amd import binding

from gpu_util import dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _keys(n, bits, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << bits, n, dtype=np.uint64)


def test_zero_spin_limit_gives_up_and_is_reported():
    n, bits = 8 << 20, 45
    keys = _keys(n, bits, 11)
    ids = np.arange(n, dtype=np.int32)
    order = np.argsort(keys, kind="stable")
    exp_k, exp_i = keys[order], ids[order]
    binding.gs_device_check()  # start from a clear error word
    prev = binding.gs_set_spin_limit(0)
    gave_up = False
    try:
        for attempt in range(3):
            k, i = dev(keys.view(np.int64)), dev(ids)
            print(f"zero-limit sort attempt {attempt}: n={n}", flush=True)
            binding.gs_sort_keys(k, i, end_bit=bits)
            try:
                binding.gs_device_check()
            except binding.GsError as e:
                assert e.status == binding.GS_ERR_DEVICE
                assert "spin limit" in str(e)
                gave_up = True
                break
            # nothing gave up on this run: the order must then be the exact one
            np.testing.assert_array_equal(host(k).view(np.uint64), exp_k)
            np.testing.assert_array_equal(host(i), exp_i)
    finally:
        binding.gs_set_spin_limit(prev)
    assert gave_up, "no partition gave up with a zero spin limit in 3 sorts of 8M keys"
    # the word was cleared by the failing check, and the default limit sorts exactly again
    binding.gs_device_check()
    k, i = dev(keys.view(np.int64)), dev(ids)
    binding.gs_sort_keys(k, i, end_bit=bits)
    binding.gs_device_check()
    np.testing.assert_array_equal(host(k).view(np.uint64), exp_k)
    np.testing.assert_array_equal(host(i), exp_i)


def test_frame_path_reports_no_error_at_the_default_limit():
    from tile_binned_gaussian_amd import synth
    from gpu_util import gpu_frame
    binding.gs_device_check()
    gpu_frame(synth.config2())
    binding.gs_device_check()
    torch.cuda.synchronize()


def test_zero_spin_limit_in_the_count_scans_is_reported():
    """Phase 1 of a 4M-splat frame (the count scan, the depth sort and the scan of the counts in depth order) at a zero
    limit: some partition gives up and the check says so; every kernel of the phase finishes and every write stays
    in its buffer (the counts and order are then meaningless and not compared, and nothing is run on them). The
    default limit then gives a whole frame with nothing to report."""
    from tile_binned_gaussian_amd import frame, synth
    from gpu_util import gpu_frame
    scene = synth.random_scene(seed=5, C=1, N=4 << 20, width=1920, height=1080, tile_size=16)
    plan = frame.FramePlan(frame.to_device(scene))
    stream = binding._stream(plan.stream)
    binding.gs_device_check()
    prev = binding.gs_set_spin_limit(0)
    gave_up = False
    try:
        for attempt in range(3):
            print(f"zero-limit phase 1 attempt {attempt}: N={scene.N}", flush=True)
            plan._count(stream)
            try:
                binding.gs_device_check(plan.stream)
            except binding.GsError as e:
                assert e.status == binding.GS_ERR_DEVICE
                assert "spin limit" in str(e)
                gave_up = True
                break
    finally:
        binding.gs_set_spin_limit(prev)
    assert gave_up, "no partition gave up with a zero spin limit in 3 runs of phase 1 over 4M splats"
    del plan
    torch.cuda.synchronize()
    binding.gs_device_check()
    gpu_frame(scene)
    binding.gs_device_check()
