"""Work on several streams: frame plans running on their own streams at the same time must each produce the
single-stream frame (every buffer a call allocates, and the growth copy of the intersection workspace, belong to
the stream its kernels run on), and binding calls on a side stream equal the same calls on the current stream.
Also: ids outside [0, C*N) in the intersection list are skipped by the composite and its backward."""
import numpy as np
import pytest
import torch

import oracle
from tile_binned_gaussian_amd import binding, frame, synth

from gpu_util import dev, host, last_splat, oracle_lists, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _assert_plan_equal(p, ref):
    n = ref.n_isects
    assert p.n_isects == n
    torch.testing.assert_close(p.keys[:n], ref.keys[:n], rtol=0, atol=0)
    torch.testing.assert_close(p.ids[:n], ref.ids[:n], rtol=0, atol=0)
    torch.testing.assert_close(p.offsets, ref.offsets, rtol=0, atol=0)
    for name in ("render_colors", "render_alphas", "render_T", "last_ids"):
        torch.testing.assert_close(getattr(p.render, name), getattr(ref.render, name), rtol=0, atol=0)


@pytest.mark.parametrize("cfg", ["config2", "config3"])
def test_frame_plans_on_concurrent_streams(cfg):
    scene = synth.CONFIGS[cfg]()
    ds = frame.to_device(scene, "cuda:0")
    ref = frame.FramePlan(ds)
    ref.run()
    torch.cuda.synchronize()
    plans = [frame.FramePlan(ds, stream=torch.cuda.Stream()) for _ in range(3)]
    for _ in range(3):
        for p in plans:  # each run queues its frame on its own stream; the host waits only for each count
            p.run()
    torch.cuda.synchronize()
    for p in plans:
        _assert_plan_equal(p, ref)


def test_binding_calls_on_a_side_stream():
    scene = synth.config2()
    ds = frame.to_device(scene, "cuda:0")
    side = torch.cuda.Stream()
    a = frame.render_frame(ds)
    side.wait_stream(torch.cuda.current_stream())  # the inputs were copied on the current stream
    b = frame.render_frame(ds, stream=side)
    torch.cuda.synchronize()
    torch.testing.assert_close(b.isect.flatten_ids, a.isect.flatten_ids, rtol=0, atol=0)
    torch.testing.assert_close(b.isect_offsets, a.isect_offsets, rtol=0, atol=0)
    torch.testing.assert_close(b.render.render_colors, a.render.render_colors, rtol=0, atol=0)
    keys = a.isect.isect_ids.clone()
    ids = a.isect.flatten_ids.clone()
    gen = torch.Generator(device="cuda").manual_seed(3)
    perm = torch.randperm(keys.numel(), generator=gen, device="cuda")
    keys, ids = keys[perm].contiguous(), ids[perm].contiguous()
    side.wait_stream(torch.cuda.current_stream())
    binding.gs_sort_keys(keys, ids, end_bit=64, stream=side)
    torch.cuda.synchronize()
    torch.testing.assert_close(keys, a.isect.isect_ids, rtol=0, atol=0)


def test_out_of_range_ids_are_skipped():
    scene = synth.random_scene(81, 2, 500, 70, 45, 16, background=True)
    fr = frame.render_frame(frame.to_device(scene, "cuda:0"))
    torch.cuda.synchronize()
    it_o, off_o = oracle_lists(scene)
    np.testing.assert_array_equal(host(fr.isect.flatten_ids), it_o.flatten_ids)
    off = off_o.reshape(-1).astype(np.int64)
    ids = it_o.flatten_ids.copy()
    n = it_o.n_isects
    rng = np.random.default_rng(82)
    bad = rng.choice(n, size=n // 7, replace=False)
    M = scene.C * scene.N
    ids[bad] = np.where(rng.uniform(size=bad.size) < 0.5, M + rng.integers(0, 1000, bad.size), -3)
    # the same frame over lists with those entries taken out
    keep = np.ones(n, bool)
    keep[bad] = False
    ends = np.append(off[1:], n)
    new_counts = np.array([keep[s:e].sum() for s, e in zip(off, ends)])
    new_off = np.concatenate([[0], np.cumsum(new_counts)[:-1]]).astype(np.int32).reshape(fr.isect_offsets.shape)
    new_ids = ids[keep]
    o = oracle.rasterize_fwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                             scene.width, scene.height, scene.tile_size, new_off, new_ids, new_ids.size,
                             scene.alpha_cutoff, scene.alpha_clamp, scene.transmittance_threshold)
    g = binding.gs_rasterize_fwd(dev(scene.means2d), dev(scene.conics), dev(scene.colors), dev(scene.opacities),
                                 dev(scene.backgrounds), scene.width, scene.height, scene.tile_size,
                                 fr.isect_offsets, dev(ids), n, scene.alpha_cutoff, scene.alpha_clamp,
                                 scene.transmittance_threshold)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(g.render_colors), o.render_colors)
    np.testing.assert_array_equal(host(g.render_T), o.render_T)
    np.testing.assert_array_equal(last_splat(host(g.last_ids), ids), last_splat(o.last_ids, new_ids))
    # the backward skips them too: the same gradients as over the lists without them
    rng2 = np.random.default_rng(83)
    gc = rng2.normal(size=o.render_colors.shape).astype(np.float32)
    ga = rng2.normal(size=o.render_alphas.shape).astype(np.float32)
    ob = oracle.rasterize_bwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                              scene.width, scene.height, scene.tile_size, new_off, new_ids, new_ids.size,
                              scene.alpha_cutoff, scene.alpha_clamp, o.render_alphas, o.last_ids, gc, ga)
    gb = binding.gs_rasterize_bwd(dev(scene.means2d), dev(scene.conics), dev(scene.colors), dev(scene.opacities),
                                  dev(scene.backgrounds), scene.width, scene.height, scene.tile_size,
                                  fr.isect_offsets, dev(ids), g.render_alphas, g.last_ids, dev(gc), dev(ga),
                                  n_isects=n, alpha_cutoff=scene.alpha_cutoff, alpha_clamp=scene.alpha_clamp)
    torch.cuda.synchronize()
    from test_gpu_backward import assert_within, summation_depth
    for field in ("means2d", "opacities", "colors", "conics"):
        assert_within(gb, ob, field, summation_depth(scene, it_o))
