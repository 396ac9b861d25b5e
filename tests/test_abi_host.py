"""Host-side checks of the C ABI (no GPU): the library loads, exports every entry point include/gs_raster.h
declares, sizes workspaces, and rejects bad arguments with the documented status before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gs_raster.h")


@pytest.fixture(scope="module")
def lib():
    from tile_binned_gaussian_amd import build, binding
    if build.stale():
        build.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gs_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_steps():
    names = declared_functions()
    for n in ("gs_isect_tiles", "gs_sort_keys", "gs_tile_ranges", "gs_rasterize_fwd", "gs_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from tile_binned_gaussian_amd import binding
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_workspace_queries(lib):
    assert lib.gs_tile_ranges_workspace_bytes() >= 4
    # sort: alternate keys + ids (12 B per pair) plus counters
    n = 13_063_842
    ws = lib.gs_sort_workspace_bytes(n, 45)
    assert 12 * n <= ws <= 12 * n + 16 * 1024 * 1024
    assert lib.gs_sort_workspace_bytes(n, 45) == lib.gs_sort_workspace_bytes(n, 47)
    assert lib.gs_isect_workspace_bytes(1, 1000, 0, 4, 4, 1) > 0
    assert lib.gs_isect_workspace_bytes(1, 1000, n, 120, 68, 1) >= ws
    assert lib.gs_isect_workspace_bytes(1, 1000, n, 120, 68, 0) < 1 << 20
    assert lib.gs_rasterize_workspace_bytes(4, 100, 67) >= 4 * 100 * 67 * 4
    assert lib.gs_isect_workspace_bytes(0, 10, 0, 4, 4, 1) == 0  # invalid -> 0


def _isect(lib, **kw):
    a = dict(means2d=None, radii=None, rpg=1, depths=None, C=1, N=0, ts=16, tw=4, th=4, sort=1, tpg=None, goff=None,
             nout=None, keys=None, ids=None, n=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.gs_isect_tiles(a["means2d"], a["radii"], a["rpg"], a["depths"], a["C"], a["N"], a["ts"], a["tw"],
                              a["th"], a["sort"], a["tpg"], a["goff"], a["nout"], a["keys"], a["ids"], a["n"], a["ws"],
                              a["wsb"], a["stream"])


def test_isect_argument_errors(lib):
    from tile_binned_gaussian_amd.binding import GS_ERR_INVALID_ARG, GS_ERR_WORKSPACE
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails on the host first
    n_out = ctypes.c_int64(0)
    assert _isect(lib, C=0) == GS_ERR_INVALID_ARG
    assert b"C >= 1" in lib.gs_last_error()
    assert _isect(lib, C=1, N=1 << 31) == GS_ERR_INVALID_ARG
    assert _isect(lib, N=4, rpg=3, means2d=fake, radii=fake, depths=fake) == GS_ERR_INVALID_ARG
    assert _isect(lib, N=4, ts=0, means2d=fake, radii=fake, depths=fake) == GS_ERR_INVALID_ARG
    assert _isect(lib, N=4, tw=0, means2d=fake, radii=fake, depths=fake) == GS_ERR_INVALID_ARG
    # 2^30 tiles (tile_bits 30) and 8 cameras (3 bits) overflow the 32 upper key bits
    assert _isect(lib, C=8, N=4, tw=1 << 16, th=1 << 14, means2d=fake, radii=fake, depths=fake,
                  goff=fake) == GS_ERR_INVALID_ARG
    assert b"exceed the 32 upper key bits" in lib.gs_last_error()
    assert _isect(lib, C=1, N=4, tw=1 << 16, th=1 << 15, means2d=fake, radii=fake, depths=fake,
                  goff=fake) == GS_ERR_INVALID_ARG
    assert b"too large" in lib.gs_last_error()
    assert _isect(lib, N=4) == GS_ERR_INVALID_ARG  # required pointers missing
    assert _isect(lib, N=4, means2d=fake, radii=fake, depths=fake, goff=fake, nout=ctypes.byref(n_out),
                  ws=None, wsb=0) == GS_ERR_INVALID_ARG  # counting needs tiles_per_gauss
    assert b"tiles_per_gauss" in lib.gs_last_error()
    assert _isect(lib, N=4, means2d=fake, radii=fake, depths=fake, goff=fake, tpg=fake, nout=ctypes.byref(n_out),
                  ws=None, wsb=0) == GS_ERR_WORKSPACE
    # the sorted count phase needs the depth-order prefix: a workspace sized for the unsorted count is too small
    small = lib.gs_isect_workspace_bytes(1, 4, 0, 4, 4, 0)
    assert small < lib.gs_isect_workspace_bytes(1, 4, 0, 4, 4, 1)
    assert _isect(lib, N=4, means2d=fake, radii=fake, depths=fake, goff=fake, tpg=fake, nout=ctypes.byref(n_out),
                  ws=fake, wsb=small, sort=1) == GS_ERR_WORKSPACE
    assert _isect(lib, C=2, N=1 << 29, means2d=fake, radii=fake, depths=fake, goff=fake, tpg=fake,
                  nout=ctypes.byref(n_out), sort=1) == GS_ERR_INVALID_ARG
    assert b"2^30 - 1 splats" in lib.gs_last_error()
    assert _isect(lib, N=4, means2d=fake, radii=fake, depths=fake, goff=fake, keys=fake, ids=fake, n=1 << 31,
                  ws=fake, wsb=1 << 40) == GS_ERR_INVALID_ARG


def test_sort_and_ranges_argument_errors(lib):
    from tile_binned_gaussian_amd.binding import GS_ERR_INVALID_ARG, GS_ERR_WORKSPACE, GS_OK
    fake = ctypes.c_void_p(0x1000)
    assert lib.gs_sort_keys(fake, fake, 1 << 30, 64, fake, 1 << 40, None) == GS_ERR_INVALID_ARG
    assert lib.gs_sort_keys(fake, fake, 10, 65, fake, 1 << 40, None) == GS_ERR_INVALID_ARG
    assert lib.gs_sort_keys(None, None, 10, 64, fake, 1 << 40, None) == GS_ERR_INVALID_ARG
    assert lib.gs_sort_keys(fake, fake, 10, 64, fake, 16, None) == GS_ERR_WORKSPACE
    assert lib.gs_sort_keys(fake, fake, 1, 64, None, 0, None) == GS_OK  # nothing to do for n < 2
    assert lib.gs_tile_ranges(fake, 10, 0, 4, 4, fake, 0, fake, 256, None) == GS_ERR_INVALID_ARG
    assert lib.gs_tile_ranges(fake, 10, 1, 4, 4, None, 0, fake, 256, None) == GS_ERR_INVALID_ARG
    assert lib.gs_tile_ranges(fake, 10, 1, 4, 4, fake, 0, None, 0, None) == GS_ERR_WORKSPACE
    assert lib.gs_tile_ranges(fake, 10, 1 << 20, 1 << 12, 1 << 4, fake, 0, fake, 256, None) == GS_ERR_INVALID_ARG


def test_rasterize_argument_errors(lib):
    from tile_binned_gaussian_amd.binding import GS_ERR_INVALID_ARG
    fake = ctypes.c_void_p(0x1000)
    F = ctypes.c_float

    def call(C=1, N=4, K=3, W=64, H=64, ts=16, tw=4, th=4, n=10, cut=1 / 255, clamp=0.99, thr=1e-4, ptr=fake):
        return lib.gs_rasterize_fwd(ptr, ptr, ptr, ptr, None, C, N, K, W, H, ts, tw, th, ptr, ptr, n, None, F(cut),
                                    F(clamp), F(thr), ptr, ptr, None, None, None, None, 0, None)
    assert call(K=0) == GS_ERR_INVALID_ARG
    assert call(K=5) == GS_ERR_INVALID_ARG
    assert call(ts=33, tw=2, th=2) == GS_ERR_INVALID_ARG
    assert call(tw=5) == GS_ERR_INVALID_ARG  # grid must be ceil(W / ts)
    assert call(W=65, tw=4) == GS_ERR_INVALID_ARG
    assert call(n=-1) == GS_ERR_INVALID_ARG
    assert call(ptr=None) == GS_ERR_INVALID_ARG
    assert call(cut=float("nan")) == GS_ERR_INVALID_ARG
    assert b"gs_rasterize_fwd" in lib.gs_last_error()


def test_rasterize_traced_argument_errors(lib):
    from tile_binned_gaussian_amd.binding import GS_ERR_INVALID_ARG
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails on the host first
    F = ctypes.c_float

    def call(S=4, L=-1, K=3, tw=4, ptr=fake):
        return lib.gs_rasterize_fwd_traced(ptr, ptr, ptr, ptr, None, 1, 4, K, 64, 64, 16, tw, 4, ptr, ptr, 10, None,
                                           F(1 / 255), F(0.99), F(1e-4), L, S, ptr, ptr, None, None, ptr, ptr,
                                           None, None, 0, None)
    assert call(S=-1) == GS_ERR_INVALID_ARG
    assert b"max_splat_steps" in lib.gs_last_error()
    assert call(K=5) == GS_ERR_INVALID_ARG
    assert b"gs_rasterize_fwd_traced" in lib.gs_last_error()
    assert call(tw=3) == GS_ERR_INVALID_ARG
    assert call(ptr=None) == GS_ERR_INVALID_ARG


def test_rasterize_bwd_argument_errors(lib):
    from tile_binned_gaussian_amd.binding import GS_ERR_INVALID_ARG
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails on the host first

    def bwd(C=1, N=4, K=3, W=32, H=32, ts=16, tw=2, th=2, n=10, cut=1 / 255, clamp=0.99, means=fake,
            ra=fake, last=fake, gc=fake, ga=fake, gm=fake):
        return lib.gs_rasterize_bwd(means, fake, fake, fake, None, C, N, K, W, H, ts, tw, th, fake, fake, n, None, cut,
                                    clamp, ra, last, gc, ga, gm, fake, fake, fake, None, None, None)

    assert bwd(K=5) == GS_ERR_INVALID_ARG
    assert b"K = 5" in lib.gs_last_error()
    assert bwd(ts=33, tw=1, th=1) == GS_ERR_INVALID_ARG
    assert bwd(tw=3) == GS_ERR_INVALID_ARG
    assert b"tile grid" in lib.gs_last_error()
    assert bwd(C=0) == GS_ERR_INVALID_ARG
    assert bwd(n=-1) == GS_ERR_INVALID_ARG
    assert bwd(ra=None) == GS_ERR_INVALID_ARG
    assert bwd(gm=None) == GS_ERR_INVALID_ARG
    assert b"NULL" in lib.gs_last_error()
    assert bwd(clamp=0.0) == GS_ERR_INVALID_ARG


def test_bins_argument_errors(lib):
    from tile_binned_gaussian_amd.binding import GS_ERR_INVALID_ARG
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails on the host first
    F = ctypes.c_float

    def bins(C=1, N=4, rpg=1, ts=16, tw=4, th=4, cap=64, ids=fake, counts=fake):
        return lib.gs_bin_tiles(fake, fake, rpg, fake, C, N, ts, tw, th, cap, ids, counts, None)
    assert bins(cap=0) == GS_ERR_INVALID_ARG
    assert bins(cap=16385) == GS_ERR_INVALID_ARG
    assert b"capacity" in lib.gs_last_error()
    assert bins(tw=1 << 12, th=1 << 12, cap=256) == GS_ERR_INVALID_ARG  # slots beyond 2^31
    assert bins(rpg=3) == GS_ERR_INVALID_ARG
    assert bins(ids=None) == GS_ERR_INVALID_ARG
    assert bins(C=0) == GS_ERR_INVALID_ARG

    def comp(cap=64, counts=fake, K=3, tw=4):
        return lib.gs_rasterize_fwd_bins(fake, fake, fake, fake, None, 1, 4, K, 64, 64, 16, tw, 4, fake, counts, cap,
                                         F(1 / 255), F(0.99), F(1e-4), fake, fake, None, None, None, None)
    assert comp(counts=None) == GS_ERR_INVALID_ARG
    assert comp(cap=0) == GS_ERR_INVALID_ARG
    assert comp(K=5) == GS_ERR_INVALID_ARG
    assert comp(tw=3) == GS_ERR_INVALID_ARG
    assert b"gs_rasterize_fwd_bins" in lib.gs_last_error()


def test_binding_rejects_counts_past_the_ids():
    """n_isects may not exceed flatten_ids' length (the kernels index ids up to n_isects); checked before any
    device work, so CPU tensors reach the check."""
    import torch
    from tile_binned_gaussian_amd import binding
    ids = torch.zeros(5, dtype=torch.int32)
    assert binding._n_isects(ids, None) == 5
    assert binding._n_isects(ids, 3) == 3
    for bad in (6, -1):
        with pytest.raises(ValueError, match="n_isects"):
            binding._n_isects(ids, bad)


def test_binding_rejects_misshapen_outputs():
    """Caller-supplied outputs must match the image batch; a wrong shape or dtype is rejected before the device
    check (the kernels would write every pixel of the declared batch)."""
    import torch
    from tile_binned_gaussian_amd import binding
    C, H, W, K = 2, 5, 7, 3
    good = binding.Render(torch.zeros((C, H, W, K)), torch.zeros((C, H, W)), torch.zeros((C, H, W)),
                          torch.zeros((C, H, W), dtype=torch.int32))
    bad_sets = [
        binding.Render(torch.zeros((C, H, W, K + 1)), good.render_alphas, good.render_T, good.last_ids),
        binding.Render(good.render_colors, torch.zeros((C, H + 1, W)), good.render_T, good.last_ids),
        binding.Render(good.render_colors, good.render_alphas, torch.zeros((C, H, W - 1)), good.last_ids),
        binding.Render(good.render_colors, good.render_alphas, good.render_T, torch.zeros((C, H, W))),
    ]
    for out in bad_sets:
        with pytest.raises((ValueError, TypeError), match="shape|must be torch"):
            binding._check_render_out(out, C, H, W, K, None)
    # the right shapes pass every shape check and stop only at the device check
    with pytest.raises(ValueError, match="GPU device"):
        binding._check_render_out(good, C, H, W, K, None)
    with pytest.raises(ValueError, match="shape"):
        binding._check_eval_counts(torch.zeros(4, dtype=torch.int64), None)
    with pytest.raises(TypeError):
        binding._check_eval_counts(torch.zeros(5, dtype=torch.int32), None)


def test_spin_limit_setter_round_trips(lib):
    """gs_set_spin_limit is host state only (no device call): it returns the previous limit."""
    prev = lib.gs_set_spin_limit(7)
    try:
        assert prev == 1 << 20
        assert lib.gs_set_spin_limit(0) == 7
    finally:
        lib.gs_set_spin_limit(prev)
