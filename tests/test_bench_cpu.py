"""Host-side logic of bench.py (no GPU): the one-GPU guard, the flop and byte models behind the
roofline figures, and how the traffic figure is read from a counter summary."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_several_gpus_are_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("B,d", [(256, 128), (64, 128), (64, 64)])
def test_flop_model_counts_the_four_products_of_a_tile(B, d):
    # one B-token tile of one head: scores Q K^T (B x d by d x B), their product with V (B x B by
    # B x d), the inter term Q KV (B x d by d x d) and the state update K^T V (d x B by B x d);
    # a product of (m x k) by (k x n) is 2 m k n flops
    products = [(B, d, B), (B, B, d), (B, d, d), (d, B, d)]
    per_tile = sum(2 * m * k * n for m, k, n in products)
    assert bench.model_flops_per_token_head(d=d, B=B) * B == per_tile


def test_byte_models():
    d, bf16, f32 = 128, 2, 4
    assert bench.BYTES_PER_TOKEN_HEAD == 4 * d * bf16            # q, k, v in; o out
    assert bench.BWD_BYTES_PER_TOKEN_HEAD == 7 * d * bf16        # q, k, v, dO in; dq, dk, dv out
    assert bench.DECODE_BYTES_PER_UNIT == 2 * d * d * f32 + 4 * d * bf16  # state in and out; q, k, v, o
    # the full-layer prefill is HBM-bound on the MI355X: its flop/byte ratio is below the ridge point
    ratio = bench.model_flops_per_token_head() / bench.BYTES_PER_TOKEN_HEAD
    assert ratio == 192
    assert ratio < bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)


def _summary(path, digest, fetch_kib, write_kib, ff, wf):
    with open(path, "w") as f:
        f.write("# counters\n")
        f.write(f"kernel_source_sha256_16 = {digest}\n")
        f.write(f"fetch_kib_per_dispatch = {fetch_kib}\nwrite_kib_per_dispatch = {write_kib}\n")
        f.write(f"copy_fetch_factor = {ff}\ncopy_write_factor = {wf}\n")
        f.write(f"traffic_bytes = {(fetch_kib * ff + write_kib * wf) * 1024}\n")


def test_traffic_is_read_only_for_the_profiled_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("full") is None                      # no summary
    path = tmp_path / "prefill_full_hbm_traffic.txt"
    _summary(path, bench.source_digest(), 1000, 500, 2.0, 1.0)
    assert bench.measured_traffic("full") == (1000 * 2.0 + 500 * 1.0) * 1024
    _summary(path, "0" * 16, 1000, 500, 2.0, 1.0)                       # kernel changed since
    assert bench.measured_traffic("full") is None
    assert bench.measured_traffic("share") is None


def test_committed_traffic_summary_is_well_formed():
    path = os.path.join(bench.PROFILES, "prefill_full_hbm_traffic.txt")
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            key, _, val = line.partition("=")
            vals[key.strip()] = val.strip()
    assert len(vals["kernel_source_sha256_16"]) == 16
    for key in ("fetch_kib_per_dispatch", "write_kib_per_dispatch", "copy_fetch_factor", "copy_write_factor",
                "traffic_bytes", "algorithmic_bytes"):
        assert float(vals[key]) > 0
    # whichever source it was taken on, the summary names the command that made it
    assert "rocprofv3 --pmc FETCH_SIZE" in open(path).read()
