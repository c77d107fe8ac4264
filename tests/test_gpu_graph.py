"""HIP graph capture of the forward through the C-ABI: the forward allocates
nothing, synchronizes nothing and records no memset, so a caller can capture it
(here with torch's graph capture on the current stream) and replay it. Every replay
is compared bit for bit with the eager forward, with eager work and host
synchronizations between the replays."""
import numpy as np
import pytest

import seeded_inputs
from helpers import to_dev, workload_inputs

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


@pytest.mark.parametrize("text_bf16", [False, True])
def test_forward_graph_replays_match_eager(af, text_bf16):
    torch = _torch()
    cfg = af.make_config(num_attention_heads=2, caption_projection_dim=512, joint_attention_dim=128,
                         pos_embed_max_size=256, num_mmdit_layers=1, num_single_dit_layers=2, max_batch=3,
                         max_latent_h=32, max_latent_w=32, max_text_len=16)
    m = af.AuraFlowModel(cfg)
    m.load_seeded_weights(seed=0)
    B, H, W, T = 3, 22, 30, 13
    lat, taus, text, mask = workload_inputs(B, 4, H, W, T, 128, lengths=seeded_inputs.valid_lengths(B, 1, T),
                                            cfg_pairs=False)
    lat_d, tau_d, text_d, mask_d = to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask)
    if text_bf16:   # a bf16 text input is staged with a device-to-device copy inside the forward
        text_d = text_d.to(torch.bfloat16)
    out = torch.empty((B, 4, H, W), dtype=torch.float32, device="cuda")
    m.forward(lat_d, tau_d, text_d, mask_d, out=out)
    torch.cuda.synchronize()
    eager = out.cpu().numpy()

    out_g = torch.empty_like(out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        m.forward(lat_d, tau_d, text_d, mask_d, out=out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.forward(lat_d, tau_d, text_d, mask_d, out=out_g)
    for i in range(4):
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out_g.cpu().numpy(), eager, err_msg=f"replay {i}")
        m.forward(lat_d, tau_d, text_d, mask_d, out=out)     # eager work between replays
        torch.cuda.synchronize()
    m.close()
