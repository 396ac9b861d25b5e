"""Seeded synthetic splat scenes: the inputs that both the HIP path and the CPU oracle consume.

This module only draws random numbers and lays them out. It holds none of the rasterizer's arithmetic
(no bounding boxes, keys, sorting, ranges or compositing), so the HIP path and the oracle can both read
its output without sharing any of the method's code.

Every array is drawn in float64 with ``numpy.random.default_rng(seed)`` (PCG64) in the order written in
each builder, then cast to float32. Conics are the inverse of a 2x2 covariance
``Sigma = R diag(l_major, l_minor) R^T`` computed in float64 and stored in the layout the gsplat
projection writes (a, b, c) = (inv00, inv01, inv11) (gsplat 1.0.0 native extension, ``projection.c``,
``gs_project_one``, conic output).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

ALPHA_CUTOFF = np.float32(1.0) / np.float32(255.0)
ALPHA_CLAMP = np.float32(0.99)
TRANSMITTANCE_THRESHOLD = np.float32(1e-4)


@dataclass
class Scene:
    """One batch of projected splats for C cameras, laid out [C, N, ...] in C order."""

    name: str
    C: int
    N: int
    width: int
    height: int
    tile_size: int
    means2d: np.ndarray  # [C, N, 2] float32
    radii: np.ndarray  # [C, N] (isotropic) or [C, N, 2] (elliptical) float32
    depths: np.ndarray  # [C, N] float32
    conics: np.ndarray  # [C, N, 3] float32
    colors: np.ndarray  # [C, N, K] float32
    opacities: np.ndarray  # [C, N] float32
    backgrounds: np.ndarray | None = None  # [C, K] float32 or None (black)
    alpha_cutoff: float = float(ALPHA_CUTOFF)
    alpha_clamp: float = float(ALPHA_CLAMP)
    transmittance_threshold: float = float(TRANSMITTANCE_THRESHOLD)
    notes: dict = field(default_factory=dict)

    @property
    def tile_width(self) -> int:
        return -(-self.width // self.tile_size)

    @property
    def tile_height(self) -> int:
        return -(-self.height // self.tile_size)

    @property
    def radii_per_gauss(self) -> int:
        return 2 if self.radii.ndim == 3 else 1

    @property
    def channels(self) -> int:
        return self.colors.shape[-1]

    @property
    def n_tiles(self) -> int:
        return self.C * self.tile_width * self.tile_height


def _conic_from_axes(l_major, l_minor, theta):
    """Covariance with eigenvalues (l_major, l_minor) rotated by theta, and its inverse (float64)."""
    cs, sn = np.cos(theta), np.sin(theta)
    sxx = l_major * cs * cs + l_minor * sn * sn
    syy = l_major * sn * sn + l_minor * cs * cs
    sxy = (l_major - l_minor) * cs * sn
    det = l_major * l_minor
    conic = np.stack([syy / det, -sxy / det, sxx / det], axis=-1)
    return sxx, syy, conic


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))


def _pack(name, C, N, W, H, ts, means, radii, depths, conics, colors, opac, notes=None, bg=None,
          elliptical=False):
    return Scene(
        name=name, C=C, N=N, width=W, height=H, tile_size=ts,
        means2d=_f32(means).reshape(C, N, 2),
        radii=_f32(radii).reshape((C, N, 2) if elliptical else (C, N)),
        depths=_f32(depths).reshape(C, N),
        conics=_f32(conics).reshape(C, N, 3),
        colors=_f32(colors).reshape(C, N, np.shape(colors)[-1]),
        opacities=_f32(opac).reshape(C, N),
        backgrounds=None if bg is None else _f32(bg).reshape(C, np.shape(bg)[-1]),
        notes=notes or {},
    )


def tiny(seed: int = 0, anisotropic: bool = False) -> Scene:
    """1 camera, 256 Gaussians, 64x64, tile 16. Isotropic radius r ~ U[1,8]; covariance eigenvalues (r/3)^2.

    With both eigenvalues equal the random rotation is a no-op; ``anisotropic=True`` draws the second
    eigenvalue as u*(r/3)^2 with u ~ U[0.1, 1] so the cross term of the conic is exercised.
    Draw order: means (N,2) U[0,64); r; theta; u (anisotropic only); depth U[0.5,10]; opacity U[0.05,0.95]; rgb.
    """
    rng = np.random.default_rng(seed)
    N, W, H = 256, 64, 64
    means = rng.uniform(0.0, 64.0, size=(N, 2))
    r = rng.uniform(1.0, 8.0, size=N)
    theta = rng.uniform(0.0, math.pi, size=N)
    l1 = (r / 3.0) ** 2
    l2 = rng.uniform(0.1, 1.0, size=N) * l1 if anisotropic else l1
    _, _, conic = _conic_from_axes(l1, l2, theta)
    depth = rng.uniform(0.5, 10.0, size=N)
    opac = rng.uniform(0.05, 0.95, size=N)
    rgb = rng.uniform(0.0, 1.0, size=(N, 3))
    return _pack("tiny-aniso" if anisotropic else "tiny", 1, N, W, H, 16, means, r, depth, conic, rgb, opac)


def config2(seed: int = 1) -> Scene:
    """1 camera, 200k Gaussians, 800x800, elliptical radii consistent with the conic.

    Draw order: means U[-40,840)^2 (5% margin); Z ~ N(0,1) -> rho = clip(4 e^Z, 0.5, 64); u ~ U[0.25,1];
    theta ~ U[0,pi); depth lognormal(ln 4, 0.5); opacity Beta(2,2); rgb U[0,1].
    sigma_major = rho/3, sigma_minor = u*sigma_major, radii = clip(3 sqrt(Sigma_axis), 0.5, 64).
    """
    rng = np.random.default_rng(seed)
    N, W, H = 200_000, 800, 800
    means = rng.uniform(-40.0, 840.0, size=(N, 2))
    rho = np.clip(4.0 * np.exp(rng.standard_normal(N)), 0.5, 64.0)
    u = rng.uniform(0.25, 1.0, size=N)
    theta = rng.uniform(0.0, math.pi, size=N)
    smaj = rho / 3.0
    sxx, syy, conic = _conic_from_axes(smaj ** 2, (u * smaj) ** 2, theta)
    radii = np.stack([np.clip(3.0 * np.sqrt(sxx), 0.5, 64.0), np.clip(3.0 * np.sqrt(syy), 0.5, 64.0)], -1)
    depth = rng.lognormal(math.log(4.0), 0.5, size=N)
    opac = rng.beta(2.0, 2.0, size=N)
    rgb = rng.uniform(0.0, 1.0, size=(N, 3))
    return _pack("config2-200k-800x800", 1, N, W, H, 16, means, radii, depth, conic, rgb, opac,
                 elliptical=True)


def _gmm_camera(rng, N, W, H, r_median, r_sigma_ln, r_max):
    """Means from a 64-component equal-weight 2D Gaussian mixture plus isotropic log-normal radii.

    Draw order: centres U over the image (64,2); s ~ U[0.02,0.08] (64); component (N); N(0,1) (N,2) for the
    offsets (std s*(W,H)); Z (N) -> r = clip(r_median e^{r_sigma_ln Z}, 0.5, r_max); u ~ U[0.25,1]; theta;
    depth lognormal(ln 4, 0.5); opacity Beta(2,5); rgb U[0,1].
    """
    centres = rng.uniform(0.0, 1.0, size=(64, 2)) * np.array([W, H], dtype=np.float64)
    s = rng.uniform(0.02, 0.08, size=64)
    comp = rng.integers(0, 64, size=N)
    z = rng.standard_normal((N, 2))
    means = centres[comp] + z * (s[comp, None] * np.array([W, H], dtype=np.float64))
    r = np.clip(r_median * np.exp(r_sigma_ln * rng.standard_normal(N)), 0.5, r_max)
    u = rng.uniform(0.25, 1.0, size=N)
    theta = rng.uniform(0.0, math.pi, size=N)
    smaj = r / 3.0
    _, _, conic = _conic_from_axes(smaj ** 2, (u * smaj) ** 2, theta)
    depth = rng.lognormal(math.log(4.0), 0.5, size=N)
    opac = rng.beta(2.0, 5.0, size=N)
    rgb = rng.uniform(0.0, 1.0, size=(N, 3))
    return means, r, conic, depth, opac, rgb


def config3(seed: int = 2, n: int = 1_000_000) -> Scene:
    """1 camera, 1M Gaussians, 1920x1080 (120x68 tiles), clustered 64-component mixture, r median 3 px."""
    rng = np.random.default_rng(seed)
    W, H = 1920, 1080
    means, r, conic, depth, opac, rgb = _gmm_camera(rng, n, W, H, 3.0, 1.8, 128.0)
    return _pack("config3-1M-1920x1080", 1, n, W, H, 16, means, r, depth, conic, rgb, opac)


def config4(seed: int = 3, n: int = 3_000_000, cameras: int = 4) -> Scene:
    """4 cameras x 3M Gaussians, 1600x1064, each camera its own mixture; 1% per camera get radius 0."""
    rng = np.random.default_rng(seed)
    W, H = 1600, 1064
    parts = [_gmm_camera(rng, n, W, H, 3.0, 1.8, 128.0) for _ in range(cameras)]
    n_zero = n // 100
    radii = []
    for c in range(cameras):
        r = parts[c][1].copy()
        r[rng.permutation(n)[:n_zero]] = 0.0
        radii.append(r)
    cat = lambda j: np.stack([p[j] for p in parts])  # noqa: E731
    return _pack("config4-4x3M-1600x1064", cameras, n, W, H, 16, cat(0), np.stack(radii), cat(3), cat(2),
                 cat(5), cat(4), notes={"zero_radius_per_camera": n_zero})


def config5(seed: int = 4, n: int = 6_000_000) -> Scene:
    """1 camera, 6M Gaussians, 3840x2160, r median 6 px; 10% exact depth duplicates; half near-zero opacity.

    Draw order: means U over the image; Z -> r = clip(6 e^{1.6 Z}, 0.5, 256); u; theta; depth lognormal(ln 4, 0.5);
    duplicate targets (permutation, first 10%) and sources (uniform over the others); opacity: a permutation's
    first half gets U[0, 1/255), the rest Beta(2,5); rgb U[0,1].
    """
    rng = np.random.default_rng(seed)
    W, H = 3840, 2160
    means = rng.uniform(0.0, 1.0, size=(n, 2)) * np.array([W, H], dtype=np.float64)
    r = np.clip(6.0 * np.exp(1.6 * rng.standard_normal(n)), 0.5, 256.0)
    u = rng.uniform(0.25, 1.0, size=n)
    theta = rng.uniform(0.0, math.pi, size=n)
    smaj = r / 3.0
    _, _, conic = _conic_from_axes(smaj ** 2, (u * smaj) ** 2, theta)
    depth = rng.lognormal(math.log(4.0), 0.5, size=n).astype(np.float32).astype(np.float64)
    n_dup = n // 10
    dst = rng.permutation(n)[:n_dup]
    src = rng.integers(0, n - 1, size=n_dup)
    src = src + (src >= dst)  # a uniformly chosen *other* Gaussian
    depth[dst] = depth[src]
    opac = rng.beta(2.0, 5.0, size=n)
    low = rng.permutation(n)[: n // 2]
    opac[low] = rng.uniform(0.0, 1.0 / 255.0, size=low.size)
    rgb = rng.uniform(0.0, 1.0, size=(n, 3))
    return _pack("config5-6M-3840x2160", 1, n, W, H, 16, means, r, depth, conic, rgb, opac,
                 notes={"duplicated_depths": n_dup, "near_zero_opacity": int(low.size)})


def random_scene(seed: int, C: int, N: int, width: int, height: int, tile_size: int = 16,
                 elliptical: bool = False, r_range=(0.5, 12.0), margin: float = 0.1,
                 zero_radius_frac: float = 0.0, dup_depth_frac: float = 0.0, channels: int = 3,
                 background: bool = False) -> Scene:
    """Small general-purpose scene for parity cases: ragged image sizes, several cameras, radius-0 splats,
    duplicated depths and optional backgrounds.

    Draw order: means U[-m*W, (1+m)*W) x U[-m*H, (1+m)*H); r ~ U[r_range]; u ~ U[0.2,1]; theta; depth U[0.5,10];
    opacity U[0.02,0.98]; colors U[0,1]; zero-radius mask; duplicate sources; background U[0,1].
    """
    rng = np.random.default_rng(seed)
    M = C * N
    means = np.stack([rng.uniform(-margin * width, (1 + margin) * width, size=M),
                      rng.uniform(-margin * height, (1 + margin) * height, size=M)], -1)
    r = rng.uniform(r_range[0], r_range[1], size=M)
    u = rng.uniform(0.2, 1.0, size=M)
    theta = rng.uniform(0.0, math.pi, size=M)
    smaj = r / 3.0
    sxx, syy, conic = _conic_from_axes(smaj ** 2, (u * smaj) ** 2, theta)
    depth = rng.uniform(0.5, 10.0, size=M).astype(np.float32).astype(np.float64)
    opac = rng.uniform(0.02, 0.98, size=M)
    rgb = rng.uniform(0.0, 1.0, size=(M, channels))
    zero = rng.uniform(size=M) < zero_radius_frac
    dup = rng.uniform(size=M) < dup_depth_frac
    src = rng.integers(0, max(M, 1), size=M)
    depth = np.where(dup, depth[src], depth)
    bg = rng.uniform(0.0, 1.0, size=(C, channels)) if background else None
    if elliptical:
        radii = np.stack([3.0 * np.sqrt(sxx), 3.0 * np.sqrt(syy)], -1)
        radii[zero] = 0.0
        radii = radii.reshape(C, N, 2)
    else:
        radii = np.where(zero, 0.0, r).reshape(C, N)
    return _pack(f"random-s{seed}-C{C}-N{N}-{width}x{height}-ts{tile_size}", C, N, width, height, tile_size,
                 means, radii, depth, conic, rgb, opac, bg=bg, elliptical=elliptical)


def lossless_radii(scene: Scene) -> np.ndarray:
    """Elliptical radii outside which no splat can reach the alpha cutoff.

    r_axis = 1.01 * sqrt(2 ln(255 o) Sigma_axis), or 0 when 255 o <= 1. Outside that extent the quadratic form
    is at least d_axis^2 / (2 Sigma_axis) (the marginal of the Gaussian), so o e^{-sigma} < 1/255.
    """
    a, b, c = (scene.conics[..., i].astype(np.float64) for i in range(3))
    det = a * c - b * b
    sxx, syy = c / det, a / det
    o = scene.opacities.astype(np.float64)
    lg = np.log(np.maximum(255.0 * o, 1e-300))
    ok = 255.0 * o > 1.0
    rx = np.where(ok, 1.01 * np.sqrt(2.0 * np.maximum(lg, 0) * sxx), 0.0)
    ry = np.where(ok, 1.01 * np.sqrt(2.0 * np.maximum(lg, 0) * syy), 0.0)
    return _f32(np.stack([rx, ry], -1))


@dataclass
class Scene3D:
    """3D Gaussians and cameras, the inputs of the EWA projection: means [N, 3], covariances [N, 3, 3] (built as
    R diag(s^2) R^T from a random unit quaternion and log-normal scales, in float64, then cast), world-to-camera
    views [C, 4, 4] and intrinsics [C, 3, 3]."""

    name: str
    means: np.ndarray
    covars: np.ndarray
    viewmats: np.ndarray
    Ks: np.ndarray
    width: int
    height: int

    @property
    def C(self) -> int:
        return self.viewmats.shape[0]

    @property
    def N(self) -> int:
        return self.means.shape[0]


def _quat_rot(q):
    w, x, y, z = (q[..., i] for i in range(4))
    return np.stack([np.stack([1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)], -1),
                     np.stack([2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)], -1),
                     np.stack([2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)], -1)], -2)


def scene3d(seed: int, N: int, C: int = 1, width: int = 1920, height: int = 1080, spread: float = 4.0,
            scale_median: float = 0.02, scale_sigma_ln: float = 1.0, distance: float = 6.0,
            behind_frac: float = 0.02, name: str | None = None) -> Scene3D:
    """Gaussians in a ball of radius `spread` around the origin (a `behind_frac` share moved behind the cameras),
    C cameras at `distance` looking at the origin from random directions, focal length 1.1 * width. Draw order:
    centres, quaternions, scales, the behind mask, then per camera its direction and roll."""
    rng = np.random.default_rng(seed)
    u = rng.normal(size=(N, 3))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    means = u * spread * rng.uniform(0, 1, (N, 1)) ** (1 / 3)
    q = rng.normal(size=(N, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    scales = scale_median * np.exp(scale_sigma_ln * rng.normal(size=(N, 3)))
    behind = rng.uniform(size=N) < behind_frac
    Rg = _quat_rot(q)
    covars = Rg @ (scales[:, :, None] ** 2 * np.transpose(Rg, (0, 2, 1)))
    views = np.zeros((C, 4, 4))
    Ks = np.zeros((C, 3, 3))
    for c in range(C):
        d = rng.normal(size=3)
        d /= np.linalg.norm(d)
        roll = rng.uniform(-0.3, 0.3)
        pos = d * distance
        fwd = -d  # camera z axis looks at the origin
        up0 = np.array([0.0, 1.0, 0.0]) if abs(fwd[1]) < 0.9 else np.array([1.0, 0.0, 0.0])
        right = np.cross(up0, fwd)
        right /= np.linalg.norm(right)
        down = np.cross(fwd, right)
        cr, sr = math.cos(roll), math.sin(roll)
        right, down = cr * right + sr * down, -sr * right + cr * down
        Rc = np.stack([right, down, fwd])  # rows: camera axes in world coordinates
        views[c, :3, :3] = Rc
        views[c, :3, 3] = -Rc @ pos
        views[c, 3, 3] = 1.0
        Ks[c] = [[1.1 * width, 0.0, width / 2], [0.0, 1.1 * width, height / 2], [0.0, 0.0, 1.0]]
    if C > 0:
        # move the `behind` share behind the first camera
        pos0 = -views[0, :3, :3].T @ views[0, :3, 3]
        means[behind] = pos0 + (pos0 - means[behind]) * 0.1
    return Scene3D(name or f"scene3d-{seed}", _f32(means), _f32(covars), _f32(views), _f32(Ks), width, height)


CONFIGS = {
    "tiny": tiny,
    "config2": config2,
    "config3": config3,
    "config4": config4,
    "config5": config5,
}
