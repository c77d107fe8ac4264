"""The allocation-free attention entry point (af_attention_noalloc: the library's
fixed per-device scratch in place of a workspace) against af_attention with a
workspace, through the C-ABI: two calls in a row, the second with a smaller
input, each equal to the workspace call bit for bit (both launch the same
kernels with the same split of the last partial round at these sizes) and to
the oracle's attention within the floating-point bar; and a call beyond the
fixed scratch is refused on the host before anything is enqueued."""
import numpy as np
import pytest

import oracle
from helpers import cosine, rel_max

pytestmark = pytest.mark.gpu

HD = 256


def _case(B, S, H, lengths, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (oracle.round_bf16(rng.standard_normal((B, S, H * HD)).astype(np.float32)) for _ in range(3))
    mask = np.ones((B, S), np.uint8)
    for b, L in enumerate(lengths):
        mask[b, 8 + L:min(S, 264)] = 0
    return q, k, v, mask


def _oracle(q, k, v, mask, H):
    B, S, D = q.shape
    heads = lambda x: x.reshape(B, S, H, HD).transpose(0, 2, 1, 3)
    eps = np.float32(1e-6)
    o = oracle.attention(oracle.layer_norm(heads(q), eps), oracle.layer_norm(heads(k), eps), heads(v), mask,
                         np.float32(1.0 / 16.0))
    return o.transpose(0, 2, 1, 3).reshape(B, S, D)


def test_noalloc_attention_two_calls_match_workspace_entry_point(af):
    import torch
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    # config B's attention shape (2 x 1288 tokens, 12 heads), then a smaller ragged one
    for (B, S, H, lengths, seed) in ((2, 1288, 12, [40, 200], 1), (1, 333, 3, [17], 2)):
        q, k, v, mask = _case(B, S, H, lengths, seed)
        qt, kt, vt = (dev(a).to(torch.bfloat16) for a in (q, k, v))
        mt = dev(mask)
        out = torch.full_like(qt, float("nan"))
        af.af_attention_noalloc(qt, kt, vt, mt, num_heads=H, out=out)
        ref_ws = af.af_attention(qt, kt, vt, mt, num_heads=H)
        torch.cuda.synchronize()
        got, want = out.float().cpu().numpy(), ref_ws.float().cpu().numpy()
        np.testing.assert_array_equal(got, want)
        ref = _oracle(q, k, v, mask, H)
        e, c = rel_max(got, ref), cosine(got, ref)
        print(f"B={B} S={S} H={H}: no-alloc == workspace entry point; vs oracle rel {e:.3e} cos {c:.6f}")
        assert e <= 2e-2 and c >= 0.999, (e, c)


def test_noalloc_attention_rejects_sizes_beyond_the_scratch(af):
    import torch
    assert af.af_attention_noalloc_max_bytes() == 64 << 20
    x = torch.zeros((2, 1793, 12 * HD), dtype=torch.bfloat16, device="cuda")      # S_pad 1920: 70.8 MB
    with pytest.raises(ValueError, match="scratch"):
        af.af_attention_noalloc(x, x, x, num_heads=12)
    y = torch.zeros((2, 1792, 12 * HD), dtype=torch.bfloat16, device="cuda")      # S_pad 1792: fits
    af.af_attention_noalloc(y, y, y, num_heads=12)
    torch.cuda.synchronize()
