"""A GTR backbone forward with random weights: 12 blocks of GLA token mixer plus
Spatial SwiGLU, for timing the library inside a whole network under a HIP graph.

GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"), Method §1: a single-scale
stack of 12 blocks over the stride-16 patch grid; each block's mixer is the
Key-only gated linear attention with a low-rank gate projection and scans in
direction LR, RL, TB, BT cycling with depth; Method §2: the feed-forward part
is a SwiGLU whose value branch is mixed on the grid by a depthwise convolution.
The pages give no widths, norms or residual layout; this module reads them as
a pre-norm residual block:

    h = RMSNorm(x);  q, k, v, z, f = h Wq, h Wk, h Wv, h Wz, h Wf   (f: rank-16 gate features)
    x = x + gla_lowrank(q, k, v, f, Wg, bg, tau, z, direction = i mod 4) Wo
    h = RMSNorm(x);  x = x + sswiglu_mix(h Win, w_conv, b_conv) Wout

The mixer (with its in-kernel gate) and the S-SwiGLU middle run in libgtrscan;
the dense projections, the patch embedding and the RMSNorms are plain torch
operations (hipBLASLt GEMMs and elementwise kernels).  Weights are seeded
random values: the network computes nothing meaningful, it has the shapes and
the work of one.
"""
from __future__ import annotations

import dataclasses
import math

import torch

from . import gla_lowrank_fwd, sswiglu_mix, PATH_AUTO


@dataclasses.dataclass(frozen=True)
class BackboneConfig:
    image: int = 640          # square input side, pixels
    patch: int = 16           # stride-16 patch embedding
    width: int = 384          # token width D = H * dk
    heads: int = 6
    dk: int = 64
    dv: int = 64
    hidden: int = 1024        # S-SwiGLU hidden size F (8/3 of the width, rounded to 64)
    rank: int = 16            # gate features
    tau: float = 16.0
    conv: int = 3             # depthwise kernel of the S-SwiGLU value branch
    blocks: int = 12
    batch: int = 1

    @property
    def grid(self) -> int:
        return self.image // self.patch


def _rmsnorm(x, w, eps=1e-5):
    xf = x.float()
    return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps) * w).to(x.dtype)


class Backbone:
    """Random-weight GTR backbone on one device (fp16 by default)."""

    def __init__(self, cfg: BackboneConfig, device, dtype=torch.float16, seed: int = 0):
        self.cfg = cfg
        self.dtype = dtype
        self.device = device
        g = torch.Generator().manual_seed(seed)

        def rnd(*shape, scale=1.0, dt=None):
            t = torch.randn(*shape, generator=g, dtype=torch.float32) * scale
            return t.to(device=device, dtype=dt or dtype)

        D, H, dk, dv, F, r = cfg.width, cfg.heads, cfg.dk, cfg.dv, cfg.hidden, cfg.rank
        self.w_patch = rnd(3 * cfg.patch * cfg.patch, D, scale=1 / math.sqrt(3 * cfg.patch ** 2))
        self.blocks = []
        for _ in range(cfg.blocks):
            s = 1 / math.sqrt(D)
            self.blocks.append(dict(
                n1=torch.ones(D, device=device), n2=torch.ones(D, device=device),
                wq=rnd(D, H * dk, scale=s), wk=rnd(D, H * dk, scale=s),
                wv=rnd(D, H * dv, scale=s), wz=rnd(D, H * dv, scale=s),
                wf=rnd(D, r, scale=s), wg=rnd(r, H * dk, scale=1 / math.sqrt(r)),
                bg=rnd(H * dk, scale=0.5, dt=torch.float32),
                rms_w=(1 + 0.1 * torch.randn(dv, generator=g)).to(device),
                wo=rnd(H * dv, D, scale=1 / math.sqrt(H * dv) / 4),
                win=rnd(D, 2 * F, scale=s),
                w_conv=rnd(F, cfg.conv, cfg.conv, scale=1 / cfg.conv, dt=torch.float32),
                b_conv=rnd(F, scale=0.1, dt=torch.float32),
                wout=rnd(F, D, scale=1 / math.sqrt(F) / 4)))

    def embed(self, image):
        """image [B, 3, S, S] -> tokens [B, gh, gw, D] (stride-16 patches, one GEMM)."""
        cfg = self.cfg
        B = image.shape[0]
        p = image.unfold(2, cfg.patch, cfg.patch).unfold(3, cfg.patch, cfg.patch)
        p = p.permute(0, 2, 3, 1, 4, 5).reshape(B, cfg.grid, cfg.grid, -1)
        return p.to(self.dtype) @ self.w_patch

    def block(self, x, i: int):
        """One block on tokens x [B, gh, gw, D]; block i scans in direction i mod 4."""
        cfg, w = self.cfg, self.blocks[i]
        B, gh, gw, D = x.shape
        H = cfg.heads
        h = _rmsnorm(x, w["n1"])
        q = (h @ w["wq"]).view(B, gh, gw, H, cfg.dk)
        k = (h @ w["wk"]).view(B, gh, gw, H, cfg.dk)
        v = (h @ w["wv"]).view(B, gh, gw, H, cfg.dv)
        z = (h @ w["wz"]).view(B, gh, gw, H, cfg.dv)
        f = h @ w["wf"]
        o, _ = gla_lowrank_fwd(q, k, v, f, w["wg"], w["bg"], cfg.tau, z, w["rms_w"], i % 4,
                               path=PATH_AUTO)
        x = x + o.view(B, gh, gw, H * cfg.dv) @ w["wo"]
        h = _rmsnorm(x, w["n2"])
        m = sswiglu_mix(h @ w["win"], w["w_conv"], w["b_conv"])
        return x + m @ w["wout"]

    def forward(self, image):
        x = self.embed(image)
        for i in range(self.cfg.blocks):
            x = self.block(x, i)
        return x
