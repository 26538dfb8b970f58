"""Host-side checks of bench.py's bookkeeping (no GPU)."""
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), ".."))
import bench  # noqa: E402


def test_code_only_strips_comments_and_whitespace():
    src = "int a; // trailing\n/* block\n comment */ int  b;\n\n  int c; // x\n"
    assert bench._code_only(src) == "int a; int b; int c;"


def test_kernel_hash_ignores_comment_edits(tmp_path, monkeypatch):
    f = tmp_path / "k.hip"
    f.write_text("__global__ void k() { int x = 1; } // one\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", [str(f)])
    h1 = bench._kernel_hash()
    f.write_text("// header\n__global__ void k() {\n  int x = 1;  /* note */\n}\n")
    assert bench._kernel_hash() == h1
    f.write_text("__global__ void k() { int x = 2; }\n")
    assert bench._kernel_hash() != h1


def test_traffic_summary_parses():
    """The committed traffic summaries (plain and gated layer) have the fields the
    bench line reads."""
    for path in (bench.TRAFFIC_FILE, bench.TRAFFIC_FILE_GATED):
        vals = {}
        for ln in open(path):
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                vals[k.strip()] = v.strip()
        assert float(vals["hbm_bytes_per_launch"]) > float(vals["algorithmic_bytes_per_launch"]) * 0.9
        assert len(vals["kernel_source_sha256_16"]) == 16


def test_gated_algorithmic_bytes():
    """The gated forward reads the decay as a bf16 pre-activation: 2 bytes per
    channel (diag) or 2 + 4 per block with the fp32 angle (rot2)."""
    from synth.gen import WORKLOADS
    L = WORKLOADS["layer"]
    per_th = (bench.algorithmic_bytes(L) - bench.algorithmic_bytes(L, gated=True)) / (L.B * L.T * L.H)
    assert per_th == 4 * L.dk - 2 * L.dk
    R = WORKLOADS["rot"]
    per_th = (bench.algorithmic_bytes(R) - bench.algorithmic_bytes(R, gated=True)) / (R.B * R.T * R.H)
    assert per_th == 4 * R.dk - 6 * (R.dk // 2)
