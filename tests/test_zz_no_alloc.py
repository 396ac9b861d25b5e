"""The allocation-free sort (gs_sort_keys_static: the library's static device scratch instead of a workspace) gives
the same bits as gs_sort_keys with a workspace, on two calls in a row, the second smaller (the scratch keeps the
first call's contents, so everything that must start at zero is cleared per call), with an even and an odd number
of digit passes; sizes above its limit are rejected before any launch."""
import numpy as np
import pytest
import torch

from tile_binned_gaussian_amd import binding

from gpu_util import dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_static_scratch_sort_matches_the_workspace_sort():
    # (pairs, key bits, seed): 45 bits = 6 digit passes, 37 bits = 5 (the odd count copies into the scratch first)
    for n, bits, seed in [(3_500_000, 45, 61), (300_000, 37, 62)]:
        rng = np.random.default_rng(seed)
        keys = rng.integers(0, 1 << bits, n, dtype=np.uint64)
        keys[rng.integers(0, n, n // 10)] = keys[0]  # ties: the stable order keeps the ids ascending
        ids = rng.permutation(n).astype(np.int32)
        print(f"static sort: n={n} bits={bits}", flush=True)
        a_k, a_i = dev(keys.view(np.int64)), dev(ids)
        b_k, b_i = dev(keys.view(np.int64)), dev(ids)
        binding.gs_sort_keys(a_k, a_i, end_bit=bits)
        binding.gs_sort_keys_static(b_k, b_i, end_bit=bits)
        torch.cuda.synchronize()
        assert torch.equal(a_k, b_k) and torch.equal(a_i, b_i)
        order = np.argsort(keys, kind="stable")
        np.testing.assert_array_equal(host(b_k).view(np.uint64), keys[order])
        np.testing.assert_array_equal(host(b_i), ids[order])
    binding.gs_device_check()


def test_static_scratch_sort_rejects_sizes_past_its_limit():
    big = (1 << 22) + 1
    k = torch.zeros(big, dtype=torch.int64, device="cuda")
    i = torch.zeros(big, dtype=torch.int32, device="cuda")
    with pytest.raises(binding.GsError) as e:
        binding.gs_sort_keys_static(k, i, end_bit=40)
    assert e.value.status == binding.GS_ERR_INVALID_ARG and "2^22" in str(e.value)
