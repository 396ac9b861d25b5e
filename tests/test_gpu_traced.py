"""GPU parity of the traced forward (gs_rasterize_fwd_traced: per-pixel trace, step cap, tile-list cap) with the
oracle's orc_rasterize_fwd_traced on the same seeded inputs and the same (bit-identical) intersection lists: colours,
alphas and T bit for bit, last ids, trace counts and every written trace entry exactly, entries past a pixel's count
unwritten; the work counter under the caps; the range backward on a capped forward against the oracle's; and the
1080p, 1M-splat frame on sampled tiles."""
import numpy as np
import pytest
import torch

import oracle
from tile_binned_gaussian_amd import binding, synth

from gpu_util import dev, gpu_frame, host, oracle_lists, require_gpu
from test_gpu_parity import SCENES

pytestmark = pytest.mark.gpu

SENTINEL = -7


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _gpu_traced(scene, fr, S, L=-1, masks=None, eval_counts=None):
    C, H, W, K = scene.C, scene.height, scene.width, scene.colors.shape[-1]
    d = torch.device("cuda")
    out = binding.TracedRender(torch.full((C, H, W, K), float("nan"), device=d),
                               torch.full((C, H, W), float("nan"), device=d),
                               torch.full((C, H, W), float("nan"), device=d),
                               torch.full((C, H, W), SENTINEL, dtype=torch.int32, device=d),
                               torch.full((C, H, W, S), SENTINEL, dtype=torch.int32, device=d),
                               torch.full((C, H, W), SENTINEL, dtype=torch.int32, device=d))
    bg = None if scene.backgrounds is None else dev(scene.backgrounds)
    binding.gs_rasterize_fwd_traced(dev(scene.means2d), dev(scene.conics), dev(scene.colors), dev(scene.opacities),
                                    bg, W, H, scene.tile_size, fr.isect_offsets, fr.isect.flatten_ids, S,
                                    max_list_entries=L, n_isects=fr.isect.n_isects, alpha_cutoff=scene.alpha_cutoff,
                                    alpha_clamp=scene.alpha_clamp,
                                    transmittance_threshold=scene.transmittance_threshold, out=out,
                                    eval_counts=eval_counts, masks=None if masks is None else dev(masks))
    torch.cuda.synchronize()
    return out


def _oracle_traced(scene, fr, S, L=-1, masks=None, tiles=None, lists=None, openmp=False):
    """The oracle's traced forward over the oracle's own lists (fr is the GPU frame, unused here: kept so both
    sides of a comparison read alike)."""
    it_o, off_o = lists if lists is not None else oracle_lists(scene)
    return oracle.rasterize_fwd_traced(scene.means2d, scene.conics, scene.colors, scene.opacities,
                                       scene.backgrounds, scene.width, scene.height, scene.tile_size, off_o,
                                       it_o.flatten_ids, it_o.n_isects, scene.alpha_cutoff, scene.alpha_clamp,
                                       scene.transmittance_threshold, S, max_list_entries=L, masks=masks,
                                       tiles=tiles, openmp=openmp)


def _assert_traced_equal(g, o, sel=(...,)):
    for name in ("render_colors", "render_alphas", "render_T", "last_ids", "trace_counts"):
        np.testing.assert_array_equal(host(getattr(g, name))[sel], getattr(o, name)[sel], err_msg=name)
    cnt = o.trace_counts[sel]
    gt, ot = host(g.trace_ids)[sel], o.trace_ids[sel]
    S = gt.shape[-1]
    written = np.arange(S) < cnt[..., None]
    np.testing.assert_array_equal(gt[written], ot[written], err_msg="trace ids")
    assert (gt[~written] == SENTINEL).all(), "entries past the count must stay unwritten"
    np.testing.assert_allclose(host(g.render_colors)[sel], o.render_colors[sel], atol=1e-4, rtol=0)


CASES = [("tiny", 8, -1), ("tiny-aniso", 2, -1), ("dense-early-out", 5, -1), ("dense-early-out", 1000, -1),
         ("multicam-ragged-elliptical", 3, 7), ("ts8-margin", 16, 2), ("ts32-ppt4", 4, -1), ("ts32-ppt4", 64, 9),
         ("ts1", 2, 1), ("deep-tiles", 12, 100), ("deep-tiles", 0, -1), ("cull-edges", 6, 0),
         ("all-equal-keys", 3, 5), ("zero-radius", 2, -1), ("one-isect", 1, -1), ("empty", 4, -1),
         ("K1", 7, -1), ("K2", 3, 11), ("K4", 9, 4)]


@pytest.mark.parametrize("name,S,L", CASES)
def test_traced_forward_matches_oracle(name, S, L):
    scene = SCENES[name]()
    fr = gpu_frame(scene)
    g = _gpu_traced(scene, fr, S, L)
    o = _oracle_traced(scene, fr, S, L)
    _assert_traced_equal(g, o)


@pytest.mark.parametrize("name", ["multicam-ragged-elliptical", "ts32-ppt4", "dense-early-out"])
def test_traced_forward_with_masks(name):
    scene = SCENES[name]()
    fr = gpu_frame(scene)
    masks = (np.random.default_rng(len(name) + 3).uniform(size=tuple(fr.isect_offsets.shape)) < 0.7).astype(np.int32)
    _assert_traced_equal(_gpu_traced(scene, fr, 6, 20, masks=masks), _oracle_traced(scene, fr, 6, 20, masks=masks))


def test_uncapped_traced_forward_equals_the_forward():
    scene = SCENES["deep-tiles"]()
    fr = gpu_frame(scene)
    g = _gpu_traced(scene, fr, 4096)
    for name in ("render_colors", "render_T", "last_ids"):
        torch.testing.assert_close(getattr(g, name), getattr(fr.render, name), rtol=0, atol=0)


@pytest.mark.parametrize("name,S,L", [("dense-early-out", 4, -1), ("ts32-ppt4", 3, 12), ("deep-tiles", 20, 50)])
def test_work_counter_under_the_caps(name, S, L):
    scene = SCENES[name]()
    fr = gpu_frame(scene)
    counts = torch.zeros(5, dtype=torch.int64, device="cuda")
    g = _gpu_traced(scene, fr, S, L, eval_counts=counts)
    o = _oracle_traced(scene, fr, S, L)
    c = host(counts)
    assert c[0] == o.n_eval
    assert c[2] == int(o.trace_counts.sum())  # composited splats = traced steps
    assert c[0] >= c[3] >= c[1] >= c[2]
    np.testing.assert_array_equal(host(g.trace_counts), o.trace_counts)


def test_backward_on_a_capped_forward_matches_oracle():
    """The range backward walks each pixel back from its last id, so on a step-capped forward's outputs it gives
    the capped forward's gradient; compared with the oracle's backward on the oracle's capped outputs."""
    from test_gpu_backward import assert_within, grads_in, summation_depth
    scene = SCENES["multicam-ragged-elliptical"]()
    fr = gpu_frame(scene)
    S = 4
    it_o, off_o = oracle_lists(scene)
    g = _gpu_traced(scene, fr, S)
    o = _oracle_traced(scene, fr, S, lists=(it_o, off_o))
    _assert_traced_equal(g, o)
    gc, ga = grads_in(scene, 21)
    ob = oracle.rasterize_bwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                              scene.width, scene.height, scene.tile_size, off_o, it_o.flatten_ids, it_o.n_isects,
                              scene.alpha_cutoff, scene.alpha_clamp, o.render_alphas, o.last_ids, gc, ga)
    gb = binding.gs_rasterize_bwd(dev(scene.means2d), dev(scene.conics), dev(scene.colors), dev(scene.opacities),
                                  dev(scene.backgrounds), scene.width, scene.height, scene.tile_size,
                                  fr.isect_offsets, fr.isect.flatten_ids, g.render_alphas, g.last_ids, dev(gc),
                                  dev(ga), n_isects=fr.isect.n_isects, alpha_cutoff=scene.alpha_cutoff,
                                  alpha_clamp=scene.alpha_clamp)
    torch.cuda.synchronize()
    adds = summation_depth(scene, it_o)
    for field in ("means2d", "conics", "colors", "opacities"):
        assert_within(gb, ob, field, adds)


def test_traced_forward_1m_splats_1080p_full_frame():
    """Every pixel of the 1M-splat frame with a 48-step cap and a 2000-entry list cap, against the oracle's traced
    forward (OpenMP build) over its own lists."""
    scene = synth.config3()
    fr = gpu_frame(scene)
    S, L = 48, 2000
    g = _gpu_traced(scene, fr, S, L)
    it_o, off_o = oracle_lists(scene, openmp=True)
    o = _oracle_traced(scene, fr, S, L, lists=(it_o, off_o), openmp=True)
    _assert_traced_equal(g, o)
    assert (o.trace_counts == S).any()  # the step cap bites on this frame
    assert (np.diff(np.append(off_o.reshape(-1), it_o.n_isects)) > L).any()  # and so does the list cap


def test_trace_rows_not_16_byte_aligned():
    """A trace buffer that starts 4 bytes past a 16-byte boundary takes the 4-byte store path; same results."""
    scene = SCENES["deep-tiles"]()
    fr = gpu_frame(scene)
    S = 8
    ref = _gpu_traced(scene, fr, S)
    C, H, W, K = scene.C, scene.height, scene.width, scene.colors.shape[-1]
    d = torch.device("cuda")
    flat = torch.full((C * H * W * S + 1,), SENTINEL, dtype=torch.int32, device=d)
    trace = flat[1:].view(C, H, W, S)
    assert trace.data_ptr() % 16 == 4
    out = binding.TracedRender(torch.empty((C, H, W, K), device=d), torch.empty((C, H, W), device=d),
                               torch.empty((C, H, W), device=d), torch.empty((C, H, W), dtype=torch.int32, device=d),
                               trace, torch.empty((C, H, W), dtype=torch.int32, device=d))
    binding.gs_rasterize_fwd_traced(dev(scene.means2d), dev(scene.conics), dev(scene.colors), dev(scene.opacities),
                                    None, W, H, scene.tile_size, fr.isect_offsets, fr.isect.flatten_ids, S,
                                    n_isects=fr.isect.n_isects, alpha_cutoff=scene.alpha_cutoff,
                                    alpha_clamp=scene.alpha_clamp,
                                    transmittance_threshold=scene.transmittance_threshold, out=out)
    torch.cuda.synchronize()
    assert int(flat[0]) == SENTINEL
    # the aligned run is itself checked against the oracle, then the unaligned one against it
    _assert_traced_equal(ref, _oracle_traced(scene, fr, S))
    torch.testing.assert_close(out.trace_counts, ref.trace_counts, rtol=0, atol=0)
    torch.testing.assert_close(out.trace_ids, ref.trace_ids, rtol=0, atol=0)
    torch.testing.assert_close(out.render_colors, ref.render_colors, rtol=0, atol=0)
