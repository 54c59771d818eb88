"""The library enqueues kernels only (no allocation, no synchronisation, no memset), so its
block forward and denoise step can be captured in a HIP graph and replayed. Each test captures
one call, then replays it several times with eager work and synchronisations in between, and
checks every replay bit for bit against the same call made eagerly."""
import numpy as np
import pytest
import torch

import synth
from oracle import sampler
from _util import binding_cfg, binding_geom, packed_block, to_dev
from test_gpu_kernels import SMALL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from video_diffusion_transformer_02_amd import binding
    binding.lib()
    return binding


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("weight", ["bf16", "i8a8"])
def test_block_forward_graph_replays_match_eager(B, weight):
    wl = SMALL.replace(weight=weight, seed_base=31)
    cfg, g = binding_cfg(wl), binding_geom(wl)
    _, pb = packed_block(wl, 0)
    mdev = torch.from_numpy(synth.modulation(wl, 0, 0)).cuda()
    x0 = to_dev(synth.storage_values(synth.normal(wl.seed_base, 5, (g.n_tokens, wl.d_model)), "bf16"), "bf16")
    ws = B.alloc_workspace(B.block_workspace_bytes(cfg, g))
    x_static = x0.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.dit_block_forward(cfg, g, pb, mdev, x_static, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        x_eager = x0.clone()
        B.dit_block_forward(cfg, g, pb, mdev, x_eager, ws)  # eager work between the replays
        torch.cuda.synchronize()
        x_static.copy_(x0)
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(x_static), _bits(x_eager), err_msg=f"replay {rep}")


def test_denoise_step_graph_replays_match_eager(B):
    """One fresh step of a two-block bf16 stack (token reduction over block 1)."""
    wl = SMALL.replace(n_blocks=2, n_steps=4, reuse=2, tr_first=1, tr_last=1, seed_base=32)
    cfg, g = binding_cfg(wl), binding_geom(wl)
    packed = [packed_block(wl, b)[1] for b in range(wl.n_blocks)]
    arr = B.block_array(packed)
    mods = torch.from_numpy(np.stack([synth.modulation(wl, 0, b) for b in range(wl.n_blocks)])).cuda()
    z0 = torch.from_numpy(synth.initial_state(wl)).cuda()
    text = to_dev(synth.storage_values(synth.text_rows(wl), "bf16"), "bf16")
    sig = sampler.sigma_grid(wl.n_steps)
    ws = B.alloc_workspace(B.step_workspace_bytes(cfg, g))

    def step(z, v):
        B.denoise_step(cfg, g, 0, wl.n_steps, wl.reuse, float(sig[0]), float(sig[1]), arr, mods, z, text, v, ws,
                       wl.tr_first, wl.tr_last)

    z_static = z0.clone()
    v_static = torch.zeros(wl.n_state, wl.d_model, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(z_static, v_static)
    torch.cuda.synchronize()
    for rep in range(3):
        z_e, v_e = z0.clone(), torch.zeros_like(v_static)
        step(z_e, v_e)
        torch.cuda.synchronize()
        z_static.copy_(z0)
        v_static.zero_()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(z_static), _bits(z_e), err_msg=f"z, replay {rep}")
        np.testing.assert_array_equal(_bits(v_static), _bits(v_e), err_msg=f"velocity cache, replay {rep}")
