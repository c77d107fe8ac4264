"""Kernel-level parity of the attention step (af_attention: QK-norm + joint
attention) against the oracle's attention on the same bf16-valued inputs.

The oracle side is oracle.layer_norm over each head of q and k followed by
oracle.attention with scale 1/16 and the key mask, in float32. At the full
1536^2 shape (S = 9480) the oracle computes sampled query rows only (every query
row is independent of the others), chosen to cover the query tiles of the last
partial round, which the launcher splits over key ranges and recombines.

Bar: the spec floating-point bar, max|d|/max|ref| <= 2e-2 and cosine >=
0.999, per case; masked-key invariance is bit-exact.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs
from helpers import cosine, rel_max

pytestmark = pytest.mark.gpu

TOL, COS = 2e-2, 0.999
HD = 256


def _inputs(B, S, H, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (oracle.round_bf16(rng.standard_normal((B, S, H * HD)).astype(np.float32)) for _ in range(3))
    return q, k, v


def _model_mask(B, S, T, lengths, R=8):
    """The forward's key pattern: R register keys, T text keys of which the first
    lengths[b] are valid, then image keys (all valid)."""
    m = np.ones((B, S), np.uint8)
    for b in range(B):
        m[b, R + lengths[b]:R + T] = 0
    return m


def _oracle(q, k, v, mask, H, rows=None):
    """fp32 oracle attention of query rows `rows` (all when None): [B, len(rows), H*256]."""
    B, S, D = q.shape
    eps = np.float32(1e-6)
    heads = lambda x: x.reshape(x.shape[0], x.shape[1], H, HD).transpose(0, 2, 1, 3)
    qs = q if rows is None else q[:, rows]
    qh = oracle.layer_norm(heads(qs), eps)
    kh = oracle.layer_norm(heads(k), eps)
    o = oracle.attention(qh, kh, heads(v), mask if mask is not None else np.ones((B, S), np.uint8),
                         np.float32(1.0 / 16.0))
    return o.transpose(0, 2, 1, 3).reshape(B, qs.shape[1], D)


def _gpu(af, q, k, v, mask, H, workspace_bytes=None):
    import torch
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    qt, kt, vt = (dev(a).to(torch.bfloat16) for a in (q, k, v))
    mt = dev(mask) if mask is not None else None
    ws = None
    if workspace_bytes is not None:
        ws = torch.empty(workspace_bytes, dtype=torch.uint8, device="cuda")
    out = af.af_attention(qt, kt, vt, mt, num_heads=H, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("B,S,H,lengths", [
    (1, 1, 1, None),            # one token
    (2, 77, 2, [3, 60]),        # ragged, one partial query tile
    (2, 300, 3, [0, 256]),      # no text key valid in sample 0 (registers and image keys remain)
    (1, 513, 1, [100]),         # one query past a tile boundary
])
def test_attention_small_matches_oracle(af, B, S, H, lengths):
    q, k, v = _inputs(B, S, H, seed=S)
    mask = None if lengths is None else _model_mask(B, S, min(256, S - 8), lengths)
    got = _gpu(af, q, k, v, mask, H)
    ref = _oracle(q, k, v, mask, H)
    e, c = rel_max(got, ref), cosine(got, ref)
    print(f"B={B} S={S} H={H}: rel {e:.3e} cos {c:.6f}")
    assert e <= TOL and c >= COS, (e, c)


def _tail_rows(S, H, B, n_cu=256, QT=128):
    """Query rows of the tiles in the last partial round ((b, h, qt) order, qt fastest)."""
    nqt = (S + QT - 1) // QT
    total = nqt * H * B
    tail = total % n_cu
    first = total - tail
    return [(t // (nqt * H), (t // nqt) % H, t % nqt) for t in range(first, total)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("lat", [128, 192])
def test_attention_full_shape_split_tail_matches_oracle(af, lat):
    """S = 8 + 256 + (lat/2)^2 (4360 at 1024^2, 9480 at 1536^2), 12 heads, CFG
    batch 2 with about half the text padded: sampled query rows, among them every
    row of one query tile that the launcher splits over key ranges, match the
    oracle; the unsplit launch (a workspace without room for partial sums) agrees
    with the split one to fp32 summation order."""
    import torch
    B, H, T = 2, 12, 256
    S = 8 + T + (lat // 2) ** 2
    q, k, v = _inputs(B, S, H, seed=lat)
    lengths = [128, 97]
    mask = _model_mask(B, S, T, lengths)
    got = _gpu(af, q, k, v, mask, H)
    tails = _tail_rows(S, H, B)
    assert tails, "this shape has a partial last round"
    b_t, h_t, qt_t = tails[-1]
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([np.arange(qt_t * 128, min(S, qt_t * 128 + 128)),
                                     rng.integers(0, S, 96), [0, 7, 8, 8 + 127, 8 + 128, S - 1]]))
    ref = _oracle(q, k, v, mask, H, rows)
    e, c = rel_max(got[:, rows], ref), cosine(got[:, rows], ref)
    head = slice(h_t * HD, (h_t + 1) * HD)
    sel = (rows >= qt_t * 128)
    et = rel_max(got[b_t, rows[sel], head], ref[b_t, sel, head])
    print(f"S={S}: sampled rows rel {e:.3e} cos {c:.6f}; split tile (b={b_t}, h={h_t}, qt={qt_t}) rel {et:.3e}")
    assert e <= TOL and c >= COS and et <= TOL, (e, c, et)
    # the same call without room for partial sums runs every tile unsplit
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    base = af.af_attention_workspace_size(B, S, H) - n_cu * (128 * 256 + 128) * 4
    unsplit = _gpu(af, q, k, v, mask, H, workspace_bytes=base)
    # both are bf16 roundings of fp32 values that differ by summation order only
    # (absolute fp32 differences of order 1e-6 of the output's scale): an element
    # differs by at most one bf16 step of the larger magnitude, so by at most
    # 2^-8 of max|out| once relative to the whole output
    diff = np.abs(unsplit - got)
    e2 = rel_max(unsplit, got)
    print(f"S={S}: unsplit vs split: {np.count_nonzero(diff)} of {diff.size} elements differ, rel {e2:.3e}")
    assert e2 <= 2.0 ** -8, e2
    # masked keys: changing k and v at excluded positions leaves the output bit-identical
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        k2[b, 8 + lengths[b]:8 + T] = 3.0
        v2[b, 8 + lengths[b]:8 + T] = -5.0
    np.testing.assert_array_equal(_gpu(af, q, k2, v2, mask, H), got)
    torch.cuda.synchronize()


def test_attention_fully_masked_sample_gives_zeros(af):
    B, S, H = 2, 70, 1
    q, k, v = _inputs(B, S, H, seed=3)
    mask = np.ones((B, S), np.uint8)
    mask[1] = 0
    got = _gpu(af, q, k, v, mask, H)
    assert np.all(got[1] == 0)
    ref = _oracle(q[:1], k[:1], v[:1], mask[:1], H)
    assert rel_max(got[:1], ref) <= TOL


def test_attention_argument_errors(af):
    import torch
    x = torch.zeros((1, 8, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        af.af_attention(x, x, x[:, :4].contiguous(), num_heads=1)          # shapes differ
    with pytest.raises(ValueError):
        af.af_attention(x.float(), x.float(), x.float(), num_heads=1)      # not bf16
    y = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        af.af_attention(y, y, y, num_heads=1)                               # head_dim 128: not built
    with pytest.raises(ValueError):
        af.af_attention(x, x, x, num_heads=1, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
