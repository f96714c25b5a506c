"""Seeded synthetic layer workloads (shapes, distributions, seeds).

This module holds no arithmetic of the method: it only draws the tensors that
the HIP path and the CPU oracle both consume (X, dY, W, an initial S), with the
shapes and value distributions of the five workloads below.  The pages train
on reasoning datasets and real Qwen-class models; neither is available, so
iid Gaussian activations and output gradients of the same layer shapes stand
in for them (iid Gaussian data is also the case the reconstruction-cosine
check of the paper's section 3.4.1 assumes).

Reading of "N(0, s)": s is the standard deviation.  Values are drawn in
float32 and rounded to bfloat16 (round to nearest even) by torch.
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Layer:
    name: str
    d: int  # output features (rows of W)
    k: int  # input features (columns of W)


@dataclass(frozen=True)
class Workload:
    key: str
    index: int  # 1-based workload number, used in the seed recipe
    title: str
    layers: tuple
    ranks: tuple
    M: int  # microbatches per step
    T: int  # tokens per microbatch
    sigma_x: float
    sigma_dy: float
    sigma_w: float = 0.02
    zero_frac: float = 0.0  # exact zeros in X (post-activation sparsity)
    heavy_frac: float = 0.0  # fraction of X rows scaled by heavy_scale (variant)
    heavy_scale: float = 50.0
    scales: tuple = (1e-5,)  # alpha * eta values of the merge
    rowadam: bool = False
    beta2: float = 0.999
    eps_rel: float = 1e-8
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload(
        key="tiny", index=1,
        title="tiny sketch d=256 k=512 r=16, 4 x 512 tokens",
        layers=(Layer("layer", 256, 512),), ranks=(16,), M=4, T=512,
        sigma_x=1.0, sigma_dy=1e-2, scales=(1e-3,),
    ),
    "attn1536": Workload(
        key="attn1536", index=2,
        title="1.5B-class attention projection d=k=1536 r=64, 8 x 4096 tokens",
        layers=(Layer("attn", 1536, 1536),), ranks=(64,), M=8, T=4096,
        sigma_x=1.0, sigma_dy=1e-3, scales=(1e-5,),
    ),
    "mlp1536": Workload(
        key="mlp1536", index=3,
        title="1.5B-class MLP up 8960x1536 / down 1536x8960 r=128, 8 x 8192 tokens, 10% zeros",
        layers=(Layer("up", 8960, 1536), Layer("down", 1536, 8960)), ranks=(128,), M=8, T=8192,
        sigma_x=1.0, sigma_dy=1e-3, zero_frac=0.1, scales=(1e-5,),
    ),
    "set7b": Workload(
        key="set7b", index=4,
        title="7B-class q/o 3584x3584, up 18944x3584, down 3584x18944, r in {64,128,256}, 16 x 8192 tokens",
        layers=(Layer("q", 3584, 3584), Layer("o", 3584, 3584), Layer("up", 18944, 3584), Layer("down", 3584, 18944)),
        ranks=(64, 128, 256), M=16, T=8192, sigma_x=1.0, sigma_dy=1e-3, scales=(1e-5,),
        rowadam=True, beta2=0.999, eps_rel=1e-8,
    ),
    "layer27b": Workload(
        key="layer27b", index=5,
        title="27B-class attention 5120x5120 and MLP 5120<->17408, r=256, 32 x 16384 tokens",
        layers=(Layer("attn", 5120, 5120), Layer("up", 17408, 5120), Layer("down", 5120, 17408)),
        ranks=(256,), M=32, T=16384, sigma_x=1.0, sigma_dy=1e-3,
        heavy_frac=0.01, heavy_scale=50.0, scales=(1e-6, 5e-6, 1e-5),
    ),
}


def seed_base(w: Workload, layer: int) -> int:
    return 1_000_000 * w.index + 10_000 * layer


def x_seed(w: Workload, layer: int, m: int) -> int:
    return seed_base(w, layer) + 2 * m


def dy_seed(w: Workload, layer: int, m: int) -> int:
    return seed_base(w, layer) + 2 * m + 1


def w_seed(w: Workload, layer: int) -> int:
    return seed_base(w, layer) + 9_999


def sign_seed(layer: int, refresh: int = 0) -> int:
    """Seed of the sign projection of layer `layer` (0-based); the tiny
    workload's single layer uses seed 0.  Successive refreshes add 100."""
    return layer + 100 * refresh


def _gen(device, seed: int):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gaussian_bf16(shape, std: float, seed: int, device="cuda", ld: int | None = None):
    """N(0, std^2) drawn in float32 with a seeded generator, rounded to bf16.
    With ``ld`` the rows live in a wider buffer (row stride ld >= shape[1])
    and the returned tensor is the left (rows, cols) view."""
    import torch

    rows, cols = shape
    width = cols if ld is None else ld
    base = torch.randn((rows, width), generator=_gen(device, seed), device=device, dtype=torch.float32)
    base.mul_(std)
    out = base.to(torch.bfloat16)
    return out[:, :cols] if width != cols else out


def layer_inputs(w: Workload, layer: int, m: int, device="cuda", T: int | None = None,
                 ld_x: int | None = None, ld_dy: int | None = None, heavy: bool = False):
    """(X_m, dY_m) of microbatch m of layer `layer`, bf16, shapes (T, k) and (T, d)."""
    import torch

    L = w.layers[layer]
    T = w.T if T is None else T
    xs = x_seed(w, layer, m)
    X = torch.randn((T, ld_x or L.k), generator=_gen(device, xs), device=device, dtype=torch.float32)
    X.mul_(w.sigma_x)
    if heavy and w.heavy_frac > 0:
        nh = int(w.heavy_frac * T)
        rows = torch.randperm(T, generator=_gen(device, dy_seed(w, layer, m) + 7000), device=device)[:nh]
        X[rows] *= w.heavy_scale
    X = X.to(torch.bfloat16)
    if w.zero_frac > 0:
        keep = torch.rand((T, ld_x or L.k), generator=_gen(device, dy_seed(w, layer, m) + 5000), device=device)
        X = torch.where(keep < w.zero_frac, torch.zeros((), dtype=X.dtype, device=device), X)
    if ld_x:
        X = X[:, : L.k]
    dY = gaussian_bf16((T, L.d), w.sigma_dy, dy_seed(w, layer, m), device=device, ld=ld_dy)
    return X, dY


def layer_weight(w: Workload, layer: int, device="cuda"):
    L = w.layers[layer]
    return gaussian_bf16((L.d, L.k), w.sigma_w, w_seed(w, layer), device=device)


def random_tensor(shape, seed: int, device="cuda", dtype=None, std: float = 1.0):
    """Generic seeded Gaussian tensor (float32 unless dtype says otherwise)."""
    import torch

    t = torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32) * std
    return t if dtype is None else t.to(dtype)


# Predicted-KL probe inputs: logits and score-change rates over a
# Qwen2.5-class vocabulary at a set of examined contexts.
KL_VOCAB = 151936
KL_CONTEXTS = 2048


def kl_inputs(n: int, V: int, seed: int, device="cuda", dtype=None, ld: int | None = None,
              z_std: float = 2.0, peak: float = 12.0, zdot_std: float = 1e-2):
    """(z, zdot), each (n, V): z ~ N(0, z_std^2) with one seeded token per row
    raised by `peak` (a peaked next-token distribution, as language-model
    logits are), zdot ~ N(0, zdot_std^2).  Drawn in float32, then cast to
    `dtype` (float32 by default).  With ``ld`` the rows live in a wider
    buffer and the returned tensors are the left (n, V) views."""
    import torch

    dtype = torch.float32 if dtype is None else dtype
    width = V if ld is None else ld
    z = torch.randn((n, width), generator=_gen(device, seed), device=device, dtype=torch.float32)
    z.mul_(z_std)
    if n and V:
        top = torch.randint(0, V, (n,), generator=_gen(device, seed + 2), device=device)
        z[torch.arange(n, device=device), top] += peak
    zd = torch.randn((n, width), generator=_gen(device, seed + 1), device=device, dtype=torch.float32)
    zd.mul_(zdot_std)
    z, zd = z.to(dtype), zd.to(dtype)
    if width != V:
        z, zd = z[:, :V], zd[:, :V]
    return z, zd
