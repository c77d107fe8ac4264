"""Host-side checks of bench.py's accounting (no GPU): the algorithmic FLOP count
the headline divides by, the per-class work the roofline uses, the hash gate on
measured HBM traffic, and the one-GPU refusal."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

D, F, L, DTXT, PATCH = 3072, 8192, 36, 2048, 16


def _fwd(B, h, w, T=256):
    nimg = (h // 2) * (w // 2)
    S = 8 + T + nimg
    return bench.forward_flops(D, F, L, B, S, T, DTXT, nimg, PATCH), S


# totals as stated to their last digit: the tolerance is half a unit of it
@pytest.mark.parametrize("B,h,w,tflop,tol", [
    (2, 128, 128, 87.93, 0.005),    # 1024^2, CFG batch 2 (the headline workload)
    (2, 192, 192, 234.12, 0.005),   # 1536^2
    (8, 128, 128, 351.7, 0.05),     # the sampling loop's batch-8 forward
])
def test_forward_flops_match_the_stated_totals(B, h, w, tflop, tol):
    flops, _ = _fwd(B, h, w)
    assert flops / 1e12 == pytest.approx(tflop, abs=tol)


def test_block_pair_flops():
    # one joint + one single block at latent 64 x 64: 1.255 TFLOP
    nimg, T = 32 * 32, 256
    S = 8 + T + nimg
    flops = bench.forward_flops(D, F, 2, 2, S, T, DTXT, nimg, PATCH)
    assert flops / 1e12 == pytest.approx(1.255, abs=0.001)


def test_class_work_sums_to_the_forward_count():
    """QKV + out-projection + FFN up + FFN down + attention per block, times 36
    blocks, plus the caption projection and the patch embed/output products,
    is the whole-forward count."""
    B, T = 2, 256
    flops, S = _fwd(B, 128, 128, T)
    per_block = sum(bench.class_work(c, D, F, B, S)[0]
                    for c in ("gemm_qkv", "gemm_out", "gemm_ffn_up", "gemm_ffn_down", "attention"))
    nimg = 64 * 64
    rest = B * (2 * T * DTXT * D + 4 * nimg * PATCH * D)
    assert L * per_block + rest == pytest.approx(flops, rel=1e-12)
    for c in ("gemm_qkv", "gemm_out", "gemm_ffn_up", "gemm_ffn_down", "attention"):
        assert bench.class_work(c, D, F, B, S)[1] == "mfma"


def test_bandwidth_class_bytes():
    B, S = 2, 4360
    ln, kind = bench.class_work("ln_modulate", D, F, B, S)
    assert kind == "hbm" and ln == B * S * D * (4 + 2)          # fp32 rows in, bf16 rows out
    mod_rows = (2 * 4 + 32) * 6 * D + 2 * D
    ada, kind = bench.class_work("adaln", D, F, B, S, mod_rows=mod_rows)
    assert kind == "hbm" and ada == 2 * (D * 256 + D * D + mod_rows * D)
    assert ada / 1e9 == pytest.approx(4.588, abs=0.001)         # bf16 weights read once


def test_mxfp8_classes_cover_every_mxfp8_product():
    # QKV, out-projection and both FFN products take MXFP8 operands in the MXFP8 model
    assert set(bench.MX_CLASSES) == {"gemm_qkv", "gemm_out", "gemm_ffn_up", "gemm_ffn_down"}


def test_measured_traffic_is_gated_by_the_source_hash(tmp_path, monkeypatch):
    text = open(os.path.join(ROOT, bench.TRAFFIC_PROFILES["gemm_ffn_up"])).read()
    fields = {}
    for line in text.splitlines():
        if line.startswith("- `") and ":" in line:
            fields[line[3:].split("`", 1)[0]] = line.split(":", 1)[1].strip().strip("`")
    assert int(fields["hbm_bytes_per_launch"]) > 0
    good = tmp_path / "good.md"
    good.write_text(text)
    bad = tmp_path / "bad.md"
    bad.write_text(text.replace(fields["source_sha256"], "0" * 64))
    monkeypatch.setattr(bench, "ROOT", ROOT)
    monkeypatch.setitem(bench.TRAFFIC_PROFILES, "gemm_ffn_up", str(good))
    got = bench.measured_traffic("gemm_ffn_up")
    # the committed summary describes the committed sources, or it reports nothing
    assert got is None or got == float(fields["hbm_bytes_per_launch"])
    monkeypatch.setitem(bench.TRAFFIC_PROFILES, "gemm_ffn_up", str(bad))
    assert bench.measured_traffic("gemm_ffn_up") is None
    assert bench.measured_traffic("no_such_class") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
