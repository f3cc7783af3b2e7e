"""The random-weight GTR backbone (gated_token_recurrence_amd.backbone) on the GPU.

1. One block against an fp64 composition of the pinned oracle pieces
   (oracle.fwd_lowrank for the mixer, oracle.sswiglu_mix for the S-SwiGLU
   middle) with numpy GEMMs and RMSNorm, rounded to fp16 wherever the GPU block
   stores an fp16 tensor.  Bar: the block's residual increment within rel-L2
   5e-3 (fp16 GEMM outputs, the mixer's 1e-3 bar and the S-SwiGLU bar compose).
2. The 12-block forward captured in a HIP graph: every replay, with eager work
   between replays, equals the eager forward bit for bit.
"""
import numpy as np
import pytest
import torch

from gated_token_recurrence_amd import backbone as bb

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def _f64(t):
    return t.detach().double().cpu().numpy()


def _rms(x, w, eps=1e-5):
    return x / np.sqrt((x * x).mean(-1, keepdims=True) + eps) * w


def test_block_matches_oracle_composition(oracle_mod):
    cfg = bb.BackboneConfig(image=16 * 20, blocks=4)
    dev = torch.device("cuda:0")
    net = bb.Backbone(cfg, dev, seed=3)
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(1, cfg.grid, cfg.grid, cfg.width, generator=g)).half().to(dev)
    r16 = lambda a: oracle_mod.round_io(a, "f16")  # noqa: E731
    for i in (0, 3):
        _note(f"backbone block {i} ({cfg.grid}x{cfg.grid}, width {cfg.width})")
        got = _f64(net.block(x, i))
        torch.cuda.synchronize()
        w = {k: _f64(v) for k, v in net.blocks[i].items()}
        xx = _f64(x)
        H, dk, dv = cfg.heads, cfg.dk, cfg.dv
        sh = xx.shape[:3]
        h = r16(_rms(xx, w["n1"]))
        q, k = r16(h @ w["wq"]).reshape(*sh, H, dk), r16(h @ w["wk"]).reshape(*sh, H, dk)
        v, z = r16(h @ w["wv"]).reshape(*sh, H, dv), r16(h @ w["wz"]).reshape(*sh, H, dv)
        f = r16(h @ w["wf"])
        o = r16(oracle_mod.fwd_lowrank(q, k, v, f, w["wg"], w["bg"], cfg.tau, z, w["rms_w"],
                                       i % 4))
        x1 = r16(xx + r16(o.reshape(*sh, H * dv) @ w["wo"]))
        h2 = r16(_rms(x1, w["n2"]))
        m = r16(oracle_mod.sswiglu_mix(r16(h2 @ w["win"]), w["w_conv"], w["b_conv"]))
        ref = r16(x1 + r16(m @ w["wout"]))
        d_got, d_ref = got - xx, ref - xx
        rel = np.linalg.norm(d_got - d_ref) / np.linalg.norm(d_ref)
        _note(f"  increment rel-L2 {rel:.2e}")
        assert np.isfinite(got).all()
        assert rel <= 5e-3, f"block {i}: increment rel-L2 {rel:.2e}"


@pytest.mark.timeout(300)
def test_graph_replay_equals_eager():
    cfg = bb.BackboneConfig()
    dev = torch.device("cuda:0")
    net = bb.Backbone(cfg, dev, seed=1)
    g = torch.Generator().manual_seed(2)
    image = torch.randn(cfg.batch, 3, cfg.image, cfg.image, generator=g).to(dev)
    stream = torch.cuda.Stream(dev)
    with torch.cuda.stream(stream):
        eager = net.forward(image).clone()   # also sizes the library's workspaces on this stream
        eager2 = net.forward(image)
    torch.cuda.synchronize()
    assert torch.equal(eager, eager2), "eager forward is not deterministic"
    assert torch.isfinite(eager.float()).all()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        out = net.forward(image)
    for rep in range(3):
        _note(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager forward"
        with torch.cuda.stream(stream):      # eager work between replays
            other = net.forward(image * 0.5)
        torch.cuda.synchronize()
        assert not torch.equal(other, eager)
